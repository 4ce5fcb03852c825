"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (per tensor): ||X_gpu - X_ref||_inf / ||X_ref||_inf <= 1e-5 on the
float32 path and <= 2e-2 on the bf16 path (float32 accumulation) for O, dQ,
dK, dV; LSE by max absolute error with the same bounds. Both sides consume the
same seeded inputs (bf16 values widened exactly to float64).

Small cases compare every element. Full-size workloads, run exactly as the
benchmark runs them (every chunk forward ascending, then the backward sweep),
compare every key's dK and dV of kv head 0 (and of the last kv head for the
32B layer) and every row's O, LSE and dQ of the first q head of those groups,
element by element; the oracle work is spread over a thread pool
(tests/oracle_pool.py).
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.selection import select_chunks
import oracle_pool as P
from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def binding():
    from sequence_chunked_exact_amd import binding as B
    return B


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_inf(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def tol(wl):
    return 1e-5 if wl.dtype == "f32" else 2e-2


def to_dev(inp):
    return {n: W.to_torch(inp.raw[n], DEV) for n in ("q", "k", "v", "do")}


def run_chunked(wl, inp, T, scale, sparse=None, ds=False):
    """Forward over all chunks, then the backward (dense chunked or sparse).

    ds: give the backward the CA_OP_BWD_DS workspace, so (bf16) the dK/dV pass
    hands dS^T to the dQ pass instead of the dQ pass recomputing it."""
    B = binding()
    t = to_dev(inp)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.chunked_forward(q, k, v, o, lse, chunk=wl.chunk, seq_len=T, softmax_scale=scale)
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    sel = None
    if sparse is None:
        B.chunked_backward(q, k, v, o, lse, do, dq, dk, dv, chunk=wl.chunk, seq_len=T, softmax_scale=scale,
                           ds_handover=ds)
    else:
        t_, seed = sparse
        sel = B.sparse_chunk_bwd(q, k, v, o, lse, do, dq, dk, dv, seq_len=T, chunk=wl.chunk, t=t_,
                                 seed=seed, softmax_scale=scale, ds_handover=ds)
    torch.cuda.synchronize()
    out = {"o": o.float().cpu().double().numpy(), "lse": lse.cpu().double().numpy(),
           "dq": dq.cpu().double().numpy(), "dk": dk.cpu().double().numpy(),
           "dv": dv.cpu().double().numpy()}
    return out, sel


def custom(name, T, C, Hq, Hkv, d, dtype, seed, scale=1.0, spike=0):
    return W.Workload(name, 1, T, C, Hq, Hkv, d, dtype, seed, softmax_scale=scale,
                      spike_rank=4 if spike else 0, spike_amp=3.0 if spike else 0.0)


def check_dense(wl, heads=None, T=None, scale=None, ds=False):
    T = wl.seq_len if T is None else T
    scale = wl.softmax_scale if scale is None else scale
    inp = W.make_inputs(wl, seq_len=T)
    note(f"[case] {wl.name} T={T} C={wl.chunk} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} d={wl.head_dim} "
         f"{wl.dtype} scale={scale:.4g} heads={heads} ds_handover={ds}")
    got, _ = run_chunked(wl, inp, T, scale, ds=ds)
    f = inp.f64
    ro, rlse = A.forward(f["q"], f["k"], f["v"], scale, heads=heads)
    rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], scale, heads=heads)
    hs = list(range(wl.n_q_heads)) if heads is None else list(heads)
    G = wl.n_q_heads // wl.n_kv_heads
    gs = sorted({h // G for h in hs})
    errs = {
        "o": rel_inf(got["o"][:, hs], ro[:, hs]),
        "lse": float(np.abs(got["lse"][:, hs] - rlse[:, hs]).max()),
        "dq": rel_inf(got["dq"][:, hs], rdq[:, hs]),
        "dk": rel_inf(got["dk"][:, gs], rdk[:, gs]),
        "dv": rel_inf(got["dv"][:, gs], rdv[:, gs]),
    }
    note(f"       errors {errs}")
    for name, e in errs.items():
        assert e <= tol(wl), (name, e)
    return errs


# ------------------------------------------------------------------ float32 path
def test_tiny_workload_every_element():
    check_dense(W.WORKLOADS["tiny"])


@pytest.mark.parametrize("T,C,Hq,Hkv,d,scale", [
    (512, 128, 4, 2, 64, 1 / 8),        # GQA, 1/sqrt(d) scale
    (300, 300, 2, 1, 64, 0.7),          # one chunk = standard backprop (D = 1)
    (200, 33, 4, 4, 128, 1.0),          # ragged chunks and tiles, d = 128
    (70, 1, 2, 2, 64, 1.0),             # one-row chunks
    (129, 64, 8, 1, 64, 0.3),           # G = 8, tail of one row
    (300, 96, 4, 2, 128, -0.6),         # negative scale (queries enter S negated)
    (150, 64, 2, 1, 64, -1.0),          # negative scale, d = 64
])
def test_f32_variants(T, C, Hq, Hkv, d, scale):
    check_dense(custom("f32_var", T, C, Hq, Hkv, d, "f32", seed=T + C, scale=scale))


# ------------------------------------------------------------------ bf16 path, reduced sizes
@pytest.mark.parametrize("name,T", [("4b_layer", 1192), ("8b_layer", 2048), ("32b_layer", 4096)])
def test_bf16_workload_shapes_reduced(name, T):
    wl = W.WORKLOADS[name]
    G = wl.n_q_heads // wl.n_kv_heads
    heads = list(range(G)) + list(range(wl.n_q_heads - G, wl.n_q_heads))   # first and last group
    check_dense(wl, heads=heads, T=T)


@pytest.mark.parametrize("T,C,Hq,Hkv,d,spike,scale", [
    (777, 100, 4, 2, 64, 0, 1.0),
    (640, 640, 4, 1, 128, 1, 1.0),
    (1000, 96, 2, 2, 128, 0, 1 / math.sqrt(128)),
    (65, 7, 2, 1, 128, 1, 1.0),
    (700, 256, 4, 2, 128, 1, -1.0),     # negative scale, spiked keys
    (333, 64, 4, 4, 64, 0, -1 / 8),     # negative scale, d = 64
])
def test_bf16_tile_and_tail_cases(T, C, Hq, Hkv, d, spike, scale):
    check_dense(custom("bf16_var", T, C, Hq, Hkv, d, "bf16", seed=T * 3 + C, scale=scale, spike=spike))


@pytest.mark.parametrize("ds", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_bf16_dkdv_launch_plan_with_six_kv_heads(d, ds):
    # Six kv heads. Both backward paths take the same key-tile plan: the
    # 2048-key prefix of chunk 0 on half-size key tiles (192 workgroups),
    # chunk 1 on full tiles (192), and chunk 2 (48 full tiles per head, 288
    # workgroups) on 42 full tiles per head followed by half-size tiles from
    # key 5376 on (72 workgroups), a split inside the chunk's own diagonal
    # block and off any multiple of the chunk size. The default backward runs
    # those as sub-grids of one launch with 192 dQ workgroups (dK/dV first in
    # chunks 0 and 1, dQ first in chunk 2; sub-grids that are not multiples of
    # the 8 XCDs come up in the randomized cases); the dS hand-over runs the
    # dK/dV pass alone, the split as two launches. 12 query heads also put the
    # forward on 64-row tiles.
    wl = custom("bf16_plan6", 6144, 2048, 12, 6, d, "bf16", seed=61 + d, spike=1)
    check_dense(wl, heads=[0, 1, 10, 11], ds=ds)


@pytest.mark.parametrize("T,C,Hq,Hkv,d,spike,scale", [
    (777, 100, 4, 2, 64, 0, 1.0),
    (1000, 96, 2, 2, 128, 1, 1 / math.sqrt(128)),
    (2048, 1024, 8, 2, 128, 1, 1.0),
    (700, 256, 4, 2, 128, 1, -1.0),     # negative scale
])
def test_bf16_ds_handover(T, C, Hq, Hkv, d, spike, scale):
    # The dS hand-over (CA_OP_BWD_DS workspace: the dK/dV pass stores dS^T and
    # the dQ pass streams it) against the oracle.
    check_dense(custom("bf16_ds", T, C, Hq, Hkv, d, "bf16", seed=T + 5 * C, scale=scale, spike=spike),
                ds=True)


@pytest.mark.parametrize("name,T", [("8b_layer", 2048), ("32b_layer", 4096)])
def test_bf16_ds_handover_workload_shapes_reduced(name, T):
    wl = W.WORKLOADS[name]
    G = wl.n_q_heads // wl.n_kv_heads
    check_dense(wl, heads=list(range(G)) + list(range(wl.n_q_heads - G, wl.n_q_heads)), T=T, ds=True)


def test_bf16_ds_and_recompute_paths_agree():
    # The two dQ passes contract bf16 dS with K; the stored dS is formed from P
    # after its rounding to bf16 (as the dK product uses it), the recomputed one
    # from float32 P, so dQ differs at the bf16 rounding level and both meet
    # the parity bar. dK, dV and the forward outputs come from the same kernels
    # and match bitwise.
    wl = custom("bf16_paths", 1500, 256, 8, 2, 128, "bf16", seed=17, spike=1)
    inp = W.make_inputs(wl)
    a, _ = run_chunked(wl, inp, 1500, 1.0, ds=True)
    b, _ = run_chunked(wl, inp, 1500, 1.0)
    for n_ in ("o", "lse", "dk", "dv"):
        assert np.array_equal(a[n_], b[n_]), n_
    f = inp.f64
    rdq, _, _ = A.backward(f["q"], f["k"], f["v"], f["do"], 1.0)
    ea, eb, ab = rel_inf(a["dq"], rdq), rel_inf(b["dq"], rdq), rel_inf(a["dq"], b["dq"])
    note(f"       dQ error: stored dS {ea:.2e}, recomputed dS {eb:.2e}; paths differ by {ab:.2e}")
    assert ea <= 2e-2 and eb <= 2e-2 and ab <= 2e-2


def test_bf16_ds_workspace_garbage_never_read():
    # The dQ pass reads only the dS^T entries the dK/dV pass wrote: fill the
    # workspace with NaN (all-ones bytes) before every chunk's backward, with
    # ragged chunks, a tail block and GQA, and the gradients stay exact.
    B = binding()
    wl = custom("bf16_nan_ws", 777, 200, 4, 2, 128, "bf16", seed=41, spike=1)
    inp = W.make_inputs(wl)
    t = to_dev(inp)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    T, C = 777, 200
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.chunked_forward(q, k, v, o, lse, chunk=C, seq_len=T)
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=C)
    ws = torch.empty(B.chunk_attn_workspace_size(desc, B.CA_OP_BWD_DS), dtype=torch.uint8, device=DEV)
    assert ws.numel() > B.chunk_attn_workspace_size(desc, B.CA_OP_BWD)   # the dS path is taken
    for i in reversed(range(-(-T // C))):
        s = i * C
        ws.fill_(255)
        B.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, chunk_start=s, chunk_len=min(C, T - s), q_row_offset=s,
                         workspace=ws)
    torch.cuda.synchronize()
    f = inp.f64
    rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], 1.0)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        g = got.cpu().double().numpy()
        assert np.isfinite(g).all(), name
        e = rel_inf(g, ref)
        note(f"       {name} error {e:.2e}")
        assert e <= 2e-2, (name, e)


# ------------------------------------------------------------------ sparse driver
def test_sparse_reduced_matches_oracle():
    wl = W.WORKLOADS["sparse_64k"]
    T, t, seed = 8192, 2, 5
    k_chunks = T // wl.chunk
    inp = W.make_inputs(wl, seq_len=T)
    note(f"[case] sparse reduced T={T} k={k_chunks} t={t} seed={seed}")
    got, sel = run_chunked(wl, inp, T, 1.0, sparse=(t, seed))
    assert sel == select_chunks(k_chunks, t, seed)
    f = inp.f64
    heads = [0, 1, 2, 3]
    rdq, rdk, rdv = A.sparse_backward(f["q"], f["k"], f["v"], f["do"], 1.0, wl.chunk, sel, k_chunks,
                                      heads=heads)
    errs = {"dq": rel_inf(got["dq"][:, heads], rdq[:, heads]),
            "dk": rel_inf(got["dk"][:, :1], rdk[:, :1]), "dv": rel_inf(got["dv"][:, :1], rdv[:, :1])}
    note(f"       errors {errs}")
    for n_, e in errs.items():
        assert e <= 2e-2, (n_, e)
    unselected = [i for i in range(k_chunks) if i not in sel]
    for i in unselected:
        assert np.all(got["dq"][:, :, i * wl.chunk:(i + 1) * wl.chunk] == 0.0)


@pytest.mark.parametrize("ds", [False, True])
def test_sparse_all_chunks_equals_chunked_backward_bitwise(ds):
    wl = custom("sp_all", 1000, 128, 4, 2, 128, "bf16", seed=21)
    inp = W.make_inputs(wl)
    dense, _ = run_chunked(wl, inp, 1000, 1.0, ds=ds)
    k_chunks = wl.n_chunks
    sparse, sel = run_chunked(wl, inp, 1000, 1.0, sparse=(k_chunks, 99), ds=ds)
    assert sel == list(range(k_chunks))
    for n_ in ("dq", "dk", "dv"):
        assert np.array_equal(dense[n_], sparse[n_]), n_


@pytest.mark.parametrize("dtype,ds", [("bf16", False), ("bf16", True), ("f32", False)])
def test_sweeps_equal_per_chunk_calls(dtype, ds):
    # chunked_fwd_sweep / chunked_bwd_sweep (the schedule computed in the
    # library) against chunk_attn_fwd / chunk_attn_bwd called chunk by chunk
    # (the schedule computed here): bitwise equal, with a ragged last chunk
    # and a grad_scale.
    B = binding()
    wl = custom("sweep", 1100, 256, 4, 2, 128, dtype, seed=13, spike=1)
    inp = W.make_inputs(wl)
    t = to_dev(inp)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    outs = []
    for lib_sweep in (True, False):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
        dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
        if lib_sweep:
            B.chunked_forward(q, k, v, o, lse, chunk=256)
            B.chunked_backward(q, k, v, o, lse, do, dq, dk, dv, chunk=256, grad_scale=0.5, ds_handover=ds)
        else:
            for i in range(wl.n_chunks):
                s_, c_ = wl.chunk_bounds(i)
                B.chunk_attn_fwd(q, k, v, o, lse, chunk_start=s_, chunk_len=c_, q_row_offset=s_)
            for i in reversed(range(wl.n_chunks)):
                s_, c_ = wl.chunk_bounds(i)
                B.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, chunk_start=s_, chunk_len=c_, q_row_offset=s_,
                                 grad_scale=0.5, ds_handover=ds)
        torch.cuda.synchronize()
        outs.append([x.float().cpu() for x in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    f = inp.f64
    rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], 1.0)
    bar = 1e-5 if dtype == "f32" else 2e-2
    for got, ref in zip(outs[0][2:], (rdq, rdk, rdv)):
        assert rel_inf(got.double().numpy(), 0.5 * ref) <= bar


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_driver_stat_slots(dtype):
    # With a CA_OP_SPARSE_BWD workspace (two slots of row statistics) each
    # chunk's launch of the drivers also computes the next chunk's statistics;
    # with only a CA_OP_BWD one they get a launch of their own per chunk. Both
    # bitwise equal, for the dense sweep and for the sparse driver (t < k,
    # ragged last chunk).
    B = binding()
    wl = custom("slots", 1000, 192, 4, 2, 128, dtype, seed=17, spike=1)
    inp = W.make_inputs(wl)
    t = to_dev(inp)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.chunked_forward(q, k, v, o, lse, chunk=192)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=192)
    one = B.chunk_attn_workspace_size(desc, B.CA_OP_BWD)
    two = B.chunk_attn_workspace_size(desc, B.CA_OP_SPARSE_BWD)
    assert two == 2 * one
    note(f"[case] driver stat slots {dtype}: {one} / {two} bytes")
    outs = {}
    for nbytes in (one, two):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        res = []
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
        dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
        B.chunked_backward(q, k, v, o, lse, do, dq, dk, dv, chunk=192, grad_scale=0.75, workspace=ws)
        res += [dq.clone(), dk.clone(), dv.clone()]
        sel = B.sparse_chunk_bwd(q, k, v, o, lse, do, dq, dk, dv, seq_len=1000, chunk=192, t=3, seed=5,
                                 workspace=ws)
        torch.cuda.synchronize()
        res += [dq.cpu(), dk.cpu(), dv.cpu()]
        outs[nbytes] = ([x.cpu() for x in res], sel)
    assert outs[one][1] == outs[two][1] == select_chunks(wl.n_chunks, 3, 5)
    for a, b_ in zip(outs[one][0], outs[two][0]):
        assert torch.equal(a, b_)
    f = inp.f64
    rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], 1.0)
    bar = 1e-5 if dtype == "f32" else 2e-2
    for got, ref in zip(outs[two][0][:3], (rdq, rdk, rdv)):
        assert rel_inf(got.double().numpy(), 0.75 * ref) <= bar
    sdq, sdk, sdv = A.sparse_backward(f["q"], f["k"], f["v"], f["do"], 1.0, 192, outs[two][1], wl.n_chunks)
    for got, ref in zip(outs[two][0][3:], (sdq, sdk, sdv)):
        assert rel_inf(got.double().numpy(), ref) <= bar


@pytest.mark.parametrize("ds", [False, True])
def test_deterministic(ds):
    wl = custom("det", 700, 256, 4, 2, 128, "bf16", seed=3)
    inp = W.make_inputs(wl)
    a, _ = run_chunked(wl, inp, 700, 1.0, ds=ds)
    b, _ = run_chunked(wl, inp, 700, 1.0, ds=ds)
    for n_ in a:
        assert np.array_equal(a[n_], b[n_]), n_


# ------------------------------------------------------------------ prefix accumulate
def test_prefix_grad_accumulate():
    B = binding()
    g = torch.Generator().manual_seed(0)
    acc = torch.randn(2, 3, 40, 128, generator=g)
    src = torch.randn(2, 3, 33, 128, generator=g)
    want = acc.double().numpy().copy()
    want[:, :, :29] += 0.375 * src.double().numpy()[:, :, :29]
    a = acc.to(DEV)
    B.prefix_grad_accumulate(a, src.to(DEV), 29, 0.375)
    torch.cuda.synchronize()
    assert np.abs(a.cpu().double().numpy() - want).max() < 1e-5


# ------------------------------------------------------------------ full sizes, bench launch config
def full_size_check(name, sparse=False, groups=(0,)):
    """The workload at full size, launched as the benchmark launches it (every
    chunk's forward ascending, then the library's sweep of the backward: all
    chunks descending, or the t drawn ones scaled by k/t). Compared element by
    element with the float64 oracle: dK and dV over every key of each kv head
    in ``groups``; O, LSE and dQ over every row of the first q head of each of
    those groups. The sum of dV over all keys of every kv head must equal the
    (scaled) sum of the dO rows that reach it."""
    wl = W.WORKLOADS[name]
    T, C, G = wl.seq_len, wl.chunk, wl.n_q_heads // wl.n_kv_heads
    note(f"[case] full size {name}: generating inputs")
    inp = W.make_inputs(wl)
    k_chunks = wl.n_chunks
    sp = (wl.sparse_t, wl.select_seed) if sparse else (k_chunks, 0)
    note(f"[case] full size {name}: GPU run")
    got, sel = run_chunked(wl, inp, T, wl.softmax_scale, sparse=sp)
    f = inp.f64
    if sparse:
        assert sel == select_chunks(k_chunks, wl.sparse_t, wl.select_seed)
    else:
        assert sel == list(range(k_chunks))
    gamma = k_chunks / len(sel)
    rows = np.concatenate([np.arange(i * C, i * C + wl.chunk_bounds(i)[1]) for i in sel])
    for g in groups:
        h = g * G
        note(f"[case] full size {name}: oracle forward of q head {h} over all {T} rows")
        ro, rlse = P.head_forward(f["q"], f["k"], f["v"], wl.softmax_scale, h)
        e_o = rel_inf(got["o"][0, h], ro)
        e_lse = float(np.abs(got["lse"][0, h] - rlse).max())
        note(f"[case] full size {name}: oracle backward of kv head {g} ({G} q heads, {rows.size} rows)")
        rdq, rdk, rdv = P.group_backward(f["q"], f["k"], f["v"], f["do"], wl.softmax_scale, g, rows=rows)
        # k/t is a power of two here (1 or 8): scaling the oracle's gradients is
        # exactly scaling its dO
        e_dq = rel_inf(got["dq"][0, h], gamma * rdq[0])
        e_dk = rel_inf(got["dk"][0, g], gamma * rdk)
        e_dv = rel_inf(got["dv"][0, g], gamma * rdv)
        note(f"       kv head {g}: o {e_o:.2e} lse {e_lse:.2e} dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
        for n_, e in (("o", e_o), ("lse", e_lse), ("dq", e_dq), ("dk", e_dk), ("dv", e_dv)):
            assert e <= 2e-2, (n_, g, e)
    if sparse:
        for i in range(k_chunks):
            if i not in sel:
                assert np.all(got["dq"][:, :, i * C:(i + 1) * C] == 0.0)
    mask = np.zeros(T, dtype=bool)
    mask[rows] = True
    want_dv = gamma * (f["do"] * mask[None, None, :, None]).reshape(
        wl.batch, wl.n_kv_heads, G, T, wl.head_dim).sum(axis=(2, 3))
    assert rel_inf(got["dv"].sum(axis=2), want_dv) <= 2e-2
    note(f"[case] full size {name}: ok")


def test_full_size_8b_layer():
    full_size_check("8b_layer")


def test_full_size_4b_layer():
    full_size_check("4b_layer")


@pytest.mark.timeout(400)
def test_full_size_32b_layer():
    full_size_check("32b_layer", groups=(0, 7))


@pytest.mark.timeout(300)
def test_full_size_sparse_64k():
    full_size_check("sparse_64k", sparse=True)
