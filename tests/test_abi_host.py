"""Host-only checks of the C ABI: exports, argument validation, selector.

No call here reaches the GPU: every rejected call returns its error code
before any device call, so fake (never dereferenced) pointers are safe.
"""
import ctypes
import os
import re

import pytest

from oracle.selection import select_chunks

b = pytest.importorskip("sequence_chunked_exact_amd.binding")
lib = b.lib
HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "chunk_attn.h")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "chunk_attn_fwd" in names and "sparse_chunk_bwd" in names
    so = ctypes.CDLL(b.LIB_PATH)
    for name in names:
        assert hasattr(so, name), name


def test_no_undeclared_c_exports():
    # Every unmangled function the library exports is one the header declares.
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]}
    c_names = {n for n in exported if not n.startswith("_")}
    assert c_names <= set(declared_functions()), sorted(c_names - set(declared_functions()))


def test_one_hip_runtime_when_loaded_before_torch():
    # A caller that imports the binding before torch must still end up with a
    # single HIP runtime in the process (the library shares torch's).
    import subprocess
    import sys
    code = ("import sequence_chunked_exact_amd.binding, torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths), sorted(paths))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, check=True)
    assert out.stdout.split()[0] == "1", out.stdout


def desc(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, kv_capacity=1024, q_capacity=256,
                q_row_offset=0, chunk_start=512, chunk_len=256, softmax_scale=1.0, dtype=b.CA_BF16)
    base.update(kw)
    return b.Desc(**base)


def fwd(d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE):
    return lib.chunk_attn_fwd(ctypes.byref(d) if d is not None else None, q, k, v, o, lse, None, 0, None)


def bwd(d, ws=FAKE, ws_bytes=1 << 20, gs=1.0, dq=FAKE):
    return lib.chunk_attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gs, dq, FAKE, FAKE,
                              ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(head_dim=96), -6),
    (dict(head_dim=256), -6),
    (dict(n_q_heads=6, n_kv_heads=4), -2),
    (dict(n_kv_heads=0), -2),
    (dict(batch=0), -2),
    (dict(chunk_len=0), -2),
    (dict(chunk_start=900), -2),            # start + len > kv_capacity
    (dict(q_row_offset=1), -2),             # offset + len > q_capacity
    (dict(chunk_start=-1), -2),
    (dict(softmax_scale=float("nan")), -2),
    (dict(softmax_scale=float("inf")), -2),
])
def test_descriptor_errors(kw, code):
    assert fwd(desc(**kw)) == code
    assert bwd(desc(**kw)) == code
    assert b.lib.chunk_attn_last_error().decode() != ""


def test_pointer_errors():
    assert fwd(None) == -1
    assert fwd(desc(), q=None) == -1
    assert fwd(desc(), lse=None) == -1
    assert fwd(desc(), v=MISALIGNED) == -4
    assert bwd(desc(), dq=MISALIGNED) == -4
    assert bwd(desc(), gs=float("nan")) == -2


def test_workspace_errors():
    d = desc()
    need = lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_BWD_MIN)
    assert need >= 4 * 4 * 256 and need % 256 == 0
    assert lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_FWD) == 0
    assert bwd(d, ws=None) == -5
    assert bwd(d, ws_bytes=need - 1) == -5
    assert bwd(d, ws=MISALIGNED, ws_bytes=need) == -4
    assert lib.chunk_attn_workspace_size(ctypes.byref(desc(head_dim=80)), b.CA_OP_BWD) == 0
    assert lib.chunk_attn_workspace_size(ctypes.byref(desc(head_dim=80)), b.CA_OP_BWD_MIN) == 0


def test_workspace_sizes_cover_the_ds_blocks():
    # bf16: CA_OP_BWD_DS adds the dS^T blocks of a chunk_len-row chunk against a
    # kv_capacity prefix (rows and keys rounded up to 128, 2 bytes each), so one
    # workspace serves every chunk of a sweep; float32 needs no more.
    for kw, rows, keys in ((dict(), 256, 1024), (dict(chunk_len=200, kv_capacity=1000), 256, 1024),
                           (dict(chunk_len=129, kv_capacity=130, q_capacity=129, chunk_start=0), 256, 256)):
        d = desc(**kw)
        lo = lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_BWD)
        full = lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_BWD_DS)
        assert full - lo == d.batch * d.n_q_heads * rows * keys * 2
        assert lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_SPARSE_BWD) == 2 * lo  # two slots
        assert lib.chunk_attn_workspace_size(ctypes.byref(d), b.CA_OP_BWD_MIN) == lo
        f32 = desc(dtype=b.CA_F32, **kw)
        assert (lib.chunk_attn_workspace_size(ctypes.byref(f32), b.CA_OP_BWD_DS)
                == lib.chunk_attn_workspace_size(ctypes.byref(f32), b.CA_OP_BWD))


def test_backward_workspace_is_bounded_by_the_chunk():
    # The backward's workspace (CA_OP_BWD; CA_OP_SPARSE_BWD holds two such
    # slots) depends only on the chunk's rows (8 bytes per row of batch * Hq *
    # C, rounded up), not on the sequence length or the capacities. 32B layer
    # (Hq 64, C 2048): 1 MiB (2 MiB) at T = 32768 and at T = 131072.
    sizes = {b.CA_OP_BWD: set(), b.CA_OP_SPARSE_BWD: set()}
    for T in (32768, 131072):
        d = desc(n_q_heads=64, n_kv_heads=8, q_capacity=T, kv_capacity=T, chunk_start=0, chunk_len=2048)
        for op in sizes:
            sizes[op].add(lib.chunk_attn_workspace_size(ctypes.byref(d), op))
    assert sizes[b.CA_OP_BWD] == {2 * 64 * 2048 * 4}
    assert sizes[b.CA_OP_SPARSE_BWD] == {2 * 2 * 64 * 2048 * 4}
    assert max(sizes[b.CA_OP_SPARSE_BWD]) <= 256 << 20


def test_accumulate_errors():
    f = lib.prefix_grad_accumulate
    assert f(None, FAKE, 1, 1, 8, 8, 64, 4, 1.0, None) == -1
    assert f(MISALIGNED, FAKE, 1, 1, 8, 8, 64, 4, 1.0, None) == -4
    assert f(FAKE, FAKE, 1, 1, 8, 8, 64, 9, 1.0, None) == -2      # prefix > capacity
    assert f(FAKE, FAKE, 1, 1, 8, 8, 6, 4, 1.0, None) == -2       # head_dim % 4
    assert f(FAKE, FAKE, 0, 1, 8, 8, 64, 4, 1.0, None) == -2


def test_sparse_errors():
    d = desc(chunk_start=0, chunk_len=128, q_capacity=1024)
    sel = (ctypes.c_int32 * 16)()
    f = lib.sparse_chunk_bwd

    def call(seq_len, t, selp=sel, ws_bytes=1 << 20):
        return f(ctypes.byref(d), seq_len, t, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 selp, FAKE, ws_bytes, None)

    assert call(1024, 9) == -2             # t > k = 8
    assert call(1024, 0) == -2
    assert call(2048, 2) == -2             # seq_len > capacity
    assert call(1024, 2, selp=None) == -1
    assert call(1024, 2, ws_bytes=16) == -5


def test_selector_matches_oracle():
    for k in (1, 3, 17, 64, 129):
        for t in sorted({1, 2, k // 3 or 1, k // 8 or 1, k}):
            if t > k:
                continue
            for seed in (0, 1, 2, 12345, 2**63 + 7, 2**64 - 1):
                assert b.chunk_select(k, t, seed) == select_chunks(k, t, seed), (k, t, seed)
    assert lib.chunk_select(4, 5, 0, (ctypes.c_int32 * 5)()) == -2
    assert lib.chunk_select(4, 1, 0, None) == -1


def test_strerror_names():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.chunk_attn_strerror(code).decode()
    assert lib.chunk_attn_strerror(-99).decode() == "unknown error"


def proj_bwd(d, dm=256, hcap=1024, hoff=512, ws=FAKE, ws_bytes=1 << 26, h=FAKE):
    return lib.qkv_proj_bwd(ctypes.byref(d), dm, hcap, hoff, h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, ws, ws_bytes, None)


def test_projection_workspace_and_errors():
    d = desc()   # bf16, Hq 4, Hkv 2, d 128, chunk 256 rows
    size = lib.qkv_proj_bwd_workspace_size
    wt = 8 * 128 * 256 * 2                            # (Hq + 2 Hkv) d x d_model, bf16
    need = size(ctypes.byref(d), 256)
    assert need == 256 * 8 * 128 * 2 + wt
    ragged = desc(chunk_len=100)  # gradient rows rounded up to 64
    assert size(ctypes.byref(ragged), 256) == 128 * 8 * 128 * 2 + wt
    assert size(ctypes.byref(desc(dtype=b.CA_F32)), 256) == 0
    assert size(ctypes.byref(d), 96) == 0             # invalid d_model
    assert proj_bwd(d, ws=None) == -5
    assert proj_bwd(d, ws_bytes=need - 1) == -5
    assert proj_bwd(d, ws=MISALIGNED, ws_bytes=need) == -4
    assert proj_bwd(d, dm=96) == -2                  # d_model not a multiple of 64
    assert proj_bwd(d, hcap=700) == -2               # h rows [512, 768) past the capacity
    assert proj_bwd(d, h=None) == -1
    assert proj_bwd(desc(head_dim=96)) == -6


def proj_bwd_wt(d, dm=256, hcap=1024, hoff=512, ws=FAKE, ws_bytes=1 << 26, wt=FAKE):
    return lib.qkv_proj_bwd_wt(ctypes.byref(d), dm, hcap, hoff, FAKE, FAKE, FAKE, FAKE, wt, FAKE, FAKE, FAKE,
                               FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_projection_transpose_sizes_and_errors():
    d = desc()   # bf16, Hq 4, Hkv 2, d 128, chunk 256 rows
    wt = 8 * 128 * 256 * 2                            # (Hq + 2 Hkv) d x d_model, bf16
    assert lib.qkv_proj_weights_t_bytes(ctypes.byref(d), 256) == wt
    assert lib.qkv_proj_weights_t_bytes(ctypes.byref(desc(dtype=b.CA_F32)), 256) == 0
    assert lib.qkv_proj_weights_t_bytes(ctypes.byref(d), 96) == 0
    grads = lib.qkv_proj_bwd_workspace_size(ctypes.byref(d), 256) - wt   # the gradient part alone
    assert grads == 256 * 8 * 128 * 2
    # the transpose: bf16 only, every pointer checked
    wtf = lib.qkv_proj_weights_t
    assert wtf(ctypes.byref(desc(dtype=b.CA_F32)), 256, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert wtf(ctypes.byref(d), 96, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert wtf(ctypes.byref(d), 256, FAKE, FAKE, FAKE, None, None) == -1
    assert wtf(ctypes.byref(d), 256, FAKE, MISALIGNED, FAKE, FAKE, None) == -4
    assert wtf(None, 256, FAKE, FAKE, FAKE, FAKE, None) == -1
    # the backward with the transpose given needs only the gradient part of the workspace
    assert proj_bwd_wt(d, ws_bytes=grads - 1) == -5
    assert proj_bwd_wt(d, ws=None) == -5
    assert proj_bwd_wt(d, wt=None) == -1              # bf16 layers need it
    assert proj_bwd_wt(d, wt=MISALIGNED) == -4
    assert proj_bwd_wt(d, dm=96) == -2
    assert proj_bwd_wt(desc(head_dim=96)) == -6
    # the backward without it still needs the whole workspace
    assert proj_bwd(d, ws_bytes=grads) == -5


def test_stack_errors():
    d = desc(chunk_start=0, chunk_len=128, q_capacity=128, n_q_heads=2, n_kv_heads=1, kv_capacity=1024)
    lay = (b.SpacoLayer * 2)()
    for i in range(2):
        for name, _ in b.SpacoLayer._fields_:
            setattr(lay[i], name, FAKE)
    sel = (ctypes.c_int32 * 3)(0, 3, 5)
    need = lib.spaco_stack_workspace_size(ctypes.byref(d), 2)
    assert need > 0
    assert lib.spaco_stack_workspace_size(ctypes.byref(d), 0) == 0

    def bwd_(seq_len=1024, L=2, layers=lay, chunks=sel, n=3, factor=2.0, ws_bytes=need, dy=FAKE, dd=d):
        return lib.spaco_stack_backward(ctypes.byref(dd), seq_len, L, layers, FAKE, dy, FAKE, 1024, chunks, n,
                                        factor, FAKE, ws_bytes, None)

    assert bwd_(L=0) == -2
    assert bwd_(layers=None) == -1
    assert bwd_(dy=None) == -1
    assert bwd_(ws_bytes=need - 1) == -5
    assert bwd_(factor=float("nan")) == -2
    assert bwd_(n=9) == -2                                    # more chunks than k = 8
    assert bwd_(chunks=(ctypes.c_int32 * 3)(0, 8, 5)) == -2   # index out of range
    assert bwd_(chunks=(ctypes.c_int32 * 3)(1, 3, 1)) == -2   # repeated
    assert bwd_(seq_len=2048) == -2                           # past the caches
    # q_capacity < C
    assert bwd_(dd=desc(chunk_len=128, q_capacity=64, n_q_heads=2, n_kv_heads=1, kv_capacity=1024)) == -2
    lay[1].dwk = None
    assert bwd_() == -1
    assert lib.spaco_stack_forward(ctypes.byref(d), 1024, 2, lay, FAKE, 1024, FAKE, need - 1, None) == -5


def test_lm_head_errors():
    HD = b.HeadDesc
    d = HD(1, 1024, 256, 1024, b.CA_BF16)
    size = lib.lm_head_sft_workspace_size
    need = size(ctypes.byref(d), 100)
    # logits (float32) + dZ (bf16, rows padded to 64) + 16 split-k partials of dH + the (max,
    # exponential sum) pairs of up to 16 segments of ps + 64 rows
    assert need == (100 * 1024 * 4 + 255) // 256 * 256 + 128 * 1024 * 2 + 16 * 100 * 256 * 4 + 164 * 16 * 2 * 4
    assert size(ctypes.byref(HD(1, 1024, 256, 1000, b.CA_BF16)), 100) == 0   # vocab % 64
    # 17 slices of 64: dH in 9 split-k parts (the last one shorter), so 9 partial slabs
    assert size(ctypes.byref(HD(1, 1024, 256, 1088, b.CA_BF16)), 100) == \
        (100 * 1088 * 4 + 255) // 256 * 256 + 128 * 1088 * 2 + 9 * 100 * 256 * 4 + 164 * 16 * 2 * 4
    assert size(ctypes.byref(d), 0) == 0

    def part(dd=d, row_start=0, rows=100, ws_bytes=need, labels=FAKE, scale=1.0):
        return lib.lm_head_sft_partition(ctypes.byref(dd), row_start, rows, FAKE, FAKE, FAKE, labels, None, scale,
                                         FAKE, FAKE, FAKE, FAKE, ws_bytes, None)

    assert part(dd=HD(1, 1024, 256, 1024, b.CA_F32)) == -6
    assert part(dd=HD(1, 1024, 96, 1024, b.CA_BF16)) == -2
    assert part(row_start=1000) == -2
    assert part(rows=0) == -2
    assert part(labels=None) == -1
    assert part(labels=MISALIGNED) == -4
    assert part(ws_bytes=need - 1) == -5
    assert part(scale=float("inf")) == -2
    assert lib.lm_head_transpose(ctypes.byref(HD(1, 1, 256, 1000, b.CA_BF16)), FAKE, FAKE, None) == -2
    assert lib.lm_head_transpose(None, FAKE, FAKE, None) == -1
    loss, c = ctypes.c_float(), ctypes.c_float()
    assert lib.lm_head_dpo_finish(ctypes.byref(d), 100, FAKE, 0.0, 0.0, 0.1, FAKE, FAKE, ctypes.byref(loss),
                                  ctypes.byref(c), None) == -2                     # batch must be 2
    assert lib.lm_head_dpo_finish(ctypes.byref(HD(2, 1024, 256, 1024, b.CA_BF16)), 100, FAKE, 0.0, 0.0, 0.1, FAKE,
                                  FAKE, None, ctypes.byref(c), None) == -1



@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles_standalone(lang, std, tmp_path):
    # The public header is self-contained C (and C++) with no HIP or torch types.
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("host compiler not available")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    src.write_text('#include "chunk_attn.h"\n'
                   'int main(void) { chunk_attn_desc d; lm_head_desc e; spaco_layer l;\n'
                   '  (void)sizeof d; (void)sizeof e; (void)sizeof l; return CA_OK; }\n')
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I",
                        os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_noalloc_backward_rejects_before_any_device_call():
    d = desc(n_q_heads=64, n_kv_heads=8, q_capacity=32768, kv_capacity=32768, chunk_start=0, chunk_len=32768)
    args = [FAKE] * 6 + [1.0] + [FAKE] * 3 + [None]
    assert lib.chunk_attn_bwd_noalloc(ctypes.byref(d), *args) == -5      # scratch too small
    assert b"static scratch" in lib.chunk_attn_last_error()
    assert lib.chunk_attn_bwd_noalloc(None, *args) == -1
    d2 = desc()
    bad = [FAKE] * 6 + [1.0] + [MISALIGNED] + [FAKE] * 2 + [None]
    assert lib.chunk_attn_bwd_noalloc(ctypes.byref(d2), *bad) == -4
    nan = [FAKE] * 6 + [float("nan")] + [FAKE] * 3 + [None]
    assert lib.chunk_attn_bwd_noalloc(ctypes.byref(d2), *nan) == -2


def test_sweep_errors():
    d = desc(chunk_start=0, chunk_len=128, q_capacity=1024, kv_capacity=1024)
    fs, bs = lib.chunked_fwd_sweep, lib.chunked_bwd_sweep
    assert fs(None, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert fs(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert fs(ctypes.byref(d), 1025, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2       # past the capacities
    assert fs(ctypes.byref(d), 1024, FAKE, MISALIGNED, FAKE, FAKE, FAKE, None) == -4
    assert fs(ctypes.byref(desc(head_dim=80)), 1024, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -6

    def bwd_(seq_len=1024, gs=1.0, ws=FAKE, ws_bytes=1 << 20, dq=FAKE):
        return bs(ctypes.byref(d), seq_len, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, gs, dq, FAKE, FAKE, ws, ws_bytes,
                  None)

    assert bwd_(seq_len=2048) == -2
    assert bwd_(gs=float("inf")) == -2
    assert bwd_(ws=None, ws_bytes=0) == -5
    assert bwd_(ws_bytes=16) == -5
    assert bwd_(dq=None) == -1


def test_bench_head_bytes_use_the_library_split_count():
    # The library's head workspace holds one float32 partial slab of dH per split-k part, so its
    # size gives the split count; bench.head_bytes must count the same number of partials.
    import importlib.util
    root = os.path.dirname(os.path.dirname(__file__))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    HD = b.HeadDesc
    ps, dm, cap = 100, 256, 1024
    for V in (64, 448, 1024, 1088, 2048, 2240, 64 * 167, 32000 // 64 * 64, 128256):
        base = (ps * V * 4 + 255) // 256 * 256 + 128 * V * 2 + 164 * 16 * 2 * 4
        need = lib.lm_head_sft_workspace_size(ctypes.byref(HD(1, cap, dm, V, b.CA_BF16)), ps)
        slab = ps * dm * 4
        lib_splits = (need - base) // slab
        assert need == base + (lib_splits * slab + 255) // 256 * 256, V
        # bench's bytes with T = ps (one partition, one dW group) minus everything but the partials
        t = bench.head_bytes(ps, dm, V, ps, 1)
        rest = 2 * V * dm * 2 + ps * dm * 2 + ps * V * 4 + ps * V * 2 + ps * V * 2 + ps * dm * 2 + 2 * V * dm * 4
        assert (t - rest) == lib_splits * ps * dm * 4, (V, lib_splits, (t - rest) // (ps * dm * 4))
