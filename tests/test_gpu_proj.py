"""GPU parity of the projection step around the chunk attention (qkv_proj_fwd /
qkv_proj_bwd through the C ABI) against the float64 oracle (oracle.projection).

Each case runs the whole chunked layer on the GPU: per chunk in ascending
order the projections then the chunk forward; then per chunk in descending
order the chunk backward then the projection backward. Q/K/V, O, the weight
gradients and the input gradient are compared element by element with the
dense oracle on the same inputs. Bars: 1e-5 on the float32 path, 2e-2 on the
bf16 path (per tensor, max error over max reference magnitude).
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import projection as P
from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-30))


def proj_bwd_wt_null(Bn, h, wq, wk, wv, q, k, dq, dk, dv, dwq, dwk, dwv, dh, s, c):
    """qkv_proj_bwd_wt called with a NULL transpose (what a float32 layer may pass)."""
    import ctypes
    desc = Bn.make_desc(q, k, chunk_start=s, chunk_len=c, q_row_offset=s)
    _, Th, dm = h.shape
    rc = Bn.lib.qkv_proj_bwd_wt(ctypes.byref(desc), dm, Th, s, h.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                                wv.data_ptr(), None, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dwq.data_ptr(),
                                dwk.data_ptr(), dwv.data_ptr(), dh.data_ptr(), None, 0, None)
    assert rc == 0, Bn.lib.chunk_attn_last_error()


def run_layer(wl, inp, transpose_once=False):
    """The chunked layer through the C ABI. transpose_once: the weights' transpose is written once
    for the backward sweep (qkv_proj_weights_t) and handed to every chunk (qkv_proj_bwd_wt); a
    float32 layer, which needs no transpose, calls qkv_proj_bwd_wt with NULL instead."""
    import torch
    from sequence_chunked_exact_amd import binding as Bn
    dev = "cuda:0"
    h, wq, wk, wv, do = (W.to_torch(inp.raw[n], dev) for n in ("h", "wq", "wk", "wv", "do"))
    B, T, dm = h.shape
    Hq, Hkv, d, C = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk
    sc = wl.softmax_scale
    dt = h.dtype
    f32 = torch.float32
    q = torch.zeros(B, Hq, T, d, dtype=dt, device=dev)
    k = torch.zeros(B, Hkv, T, d, dtype=dt, device=dev)
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=f32, device=dev)
    starts = list(range(0, T, C))
    for s in starts:
        c = min(C, T - s)
        Bn.qkv_proj_fwd(h, wq, wk, wv, q, k, v, chunk_start=s, chunk_len=c, q_row_offset=s)
        Bn.chunk_attn_fwd(q, k, v, o, lse, chunk_start=s, chunk_len=c, q_row_offset=s, softmax_scale=sc)
    dq = torch.zeros(B, Hq, T, d, dtype=f32, device=dev)
    dk = torch.zeros(B, Hkv, T, d, dtype=f32, device=dev)
    dv = torch.zeros_like(dk)
    dwq = torch.zeros(dm, Hq * d, dtype=f32, device=dev)
    dwk = torch.zeros(dm, Hkv * d, dtype=f32, device=dev)
    dwv = torch.zeros_like(dwk)
    dh = torch.full((B, T, dm), float("nan"), dtype=f32, device=dev)
    f32_layer = dt == torch.float32
    wcat_t = Bn.qkv_proj_weights_t(wq, wk, wv, q, k) if transpose_once and not f32_layer else None
    for s in reversed(starts):
        c = min(C, T - s)
        print(f"[case] {wl.name} chunk {s // C} bwd", flush=True)
        Bn.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, chunk_start=s, chunk_len=c, q_row_offset=s,
                          softmax_scale=sc)
        if transpose_once and f32_layer:
            proj_bwd_wt_null(Bn, h, wq, wk, wv, q, k, dq, dk, dv, dwq, dwk, dwv, dh, s, c)
        else:
            Bn.qkv_proj_bwd(h, wq, wk, wv, q, k, dq, dk, dv, dwq, dwk, dwv, dh, chunk_start=s, chunk_len=c,
                            q_row_offset=s, w_cat_t=wcat_t)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().numpy().astype(np.float64)
           for n, t in dict(q=q, k=k, v=v, o=o, dwq=dwq, dwk=dwk, dwv=dwv, dh=dh).items()}
    return out


CASES = [
    # name, B, T, C, d_model, Hq, Hkv, d, dtype
    ("f32_small_ragged", 1, 256, 96, 128, 4, 2, 64, "f32"),
    ("f32_min_dmodel_one_chunk", 1, 100, 100, 64, 2, 1, 64, "f32"),
    ("bf16_batch2_ragged", 2, 640, 250, 256, 4, 2, 128, "bf16"),
    ("bf16_8b_dims_T2048", 1, 2048, 1024, 4096, 32, 8, 128, "bf16"),
    # Q|K|V widths 192/64/64: output and weight tiles straddle the three
    # projections; d_model 192 leaves a partial weight-gradient tile
    ("bf16_d64_one_kv_head", 1, 300, 70, 192, 3, 1, 64, "bf16"),
    # d_model 64 (one partial tile), 7-row chunks (padded to 64), batch 2
    ("bf16_min_dmodel_tiny_chunks", 2, 40, 7, 64, 2, 2, 64, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_parity(case):
    name, B, T, C, dm, Hq, Hkv, d, dtype = case
    print(f"[case] {name}", flush=True)
    wl = W.LayerWorkload(name, B, T, C, dm, Hq, Hkv, d, dtype, seed=13)
    inp = W.make_layer_inputs(wl)
    got = run_layer(wl, inp)
    f = inp.f64
    qr, kr, vr = P.qkv_forward(f["h"], f["wq"], f["wk"], f["wv"], Hq, Hkv)
    orf, _ = A.forward(qr, kr, vr, wl.softmax_scale)
    dwq, dwk, dwv, dh = P.layer_backward(f["h"], f["wq"], f["wk"], f["wv"], f["do"], Hq, Hkv, wl.softmax_scale)
    tol = 1e-5 if dtype == "f32" else 2e-2
    errs = {"q": rel(got["q"], qr), "k": rel(got["k"], kr), "v": rel(got["v"], vr), "o": rel(got["o"], orf),
            "dwq": rel(got["dwq"], dwq), "dwk": rel(got["dwk"], dwk), "dwv": rel(got["dwv"], dwv),
            "dh": rel(got["dh"], dh)}
    print(name, {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n_, e in errs.items():
        assert e <= tol, (n_, e)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_weights_transposed_once(case):
    """qkv_proj_bwd_wt with the transpose written once per sweep gives qkv_proj_bwd's results bit for
    bit (the same kernels read the same W_cat^T), over ragged sweeps, batch 2 and the 8B dims; for
    float32 layers, called with a NULL transpose, it is qkv_proj_bwd."""
    name, B, T, C, dm, Hq, Hkv, d, dtype = case
    print(f"[case] {name} transpose once", flush=True)
    wl = W.LayerWorkload(name, B, T, C, dm, Hq, Hkv, d, dtype, seed=13)
    inp = W.make_layer_inputs(wl)
    a = run_layer(wl, inp)
    b_ = run_layer(wl, inp, transpose_once=True)
    for n_ in a:
        assert np.array_equal(a[n_], b_[n_]), n_


def test_layer_full_size_sampled():
    """The 8B attention layer at full size (T = 16384, d_model 4096, C = 1024),
    run exactly as the layer benchmark runs it. Checked on samples the oracle
    can compute one by one: Q/K/V rows (H_in rows times the weights), and the
    projection backward from the float32 gradients the GPU's attention
    backward produced: dH_in rows and single weight-gradient entries
    (sum over all T positions)."""
    import torch
    from sequence_chunked_exact_amd import binding as Bn
    wl = W.LAYER_WORKLOADS["8b_attn_layer"]
    print(f"[case] {wl.name} full size", flush=True)
    inp = W.make_layer_inputs(wl, keep_f64=False)
    dev = "cuda:0"
    h, wq, wk, wv, do = (W.to_torch(inp.raw[n], dev) for n in ("h", "wq", "wk", "wv", "do"))
    B, T, dm = h.shape
    Hq, Hkv, d, C = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk
    f32 = torch.float32
    q = torch.zeros(B, Hq, T, d, dtype=h.dtype, device=dev)
    k = torch.zeros(B, Hkv, T, d, dtype=h.dtype, device=dev)
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=f32, device=dev)
    dq = torch.zeros(B, Hq, T, d, dtype=f32, device=dev)
    dk = torch.zeros(B, Hkv, T, d, dtype=f32, device=dev)
    dv = torch.zeros_like(dk)
    dwq = torch.zeros(dm, Hq * d, dtype=f32, device=dev)
    dwk = torch.zeros(dm, Hkv * d, dtype=f32, device=dev)
    dwv = torch.zeros_like(dwk)
    dh = torch.full((B, T, dm), float("nan"), dtype=f32, device=dev)
    starts = list(range(0, T, C))
    for s in starts:
        Bn.qkv_proj_fwd(h, wq, wk, wv, q, k, v, chunk_start=s, chunk_len=min(C, T - s), q_row_offset=s)
        Bn.chunk_attn_fwd(q, k, v, o, lse, chunk_start=s, chunk_len=min(C, T - s), q_row_offset=s,
                          softmax_scale=wl.softmax_scale)
    for s in reversed(starts):
        c = min(C, T - s)
        Bn.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, chunk_start=s, chunk_len=c, q_row_offset=s,
                          softmax_scale=wl.softmax_scale)
        Bn.qkv_proj_bwd(h, wq, wk, wv, q, k, dq, dk, dv, dwq, dwk, dwv, dh, chunk_start=s, chunk_len=c,
                        q_row_offset=s)
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f64(inp.raw["h"])[0]
    wf = {n: W.bf16_bits_to_f64(inp.raw[n]) for n in ("wq", "wk", "wv")}
    g = {"wq": P.heads_to_cols(dq.cpu().double().numpy())[0], "wk": P.heads_to_cols(dk.cpu().double().numpy())[0],
         "wv": P.heads_to_cols(dv.cpu().double().numpy())[0]}
    assert all(np.isfinite(x).all() for x in g.values())
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, C - 1, C, T - 1], rng.integers(0, T, 12)]))
    out = {"wq": P.heads_to_cols(q.float().cpu().double().numpy())[0],
           "wk": P.heads_to_cols(k.float().cpu().double().numpy())[0],
           "wv": P.heads_to_cols(v.float().cpu().double().numpy())[0]}
    for n_ in ("wq", "wk", "wv"):
        ref = hf[rows] @ wf[n_]
        e = rel(out[n_][rows], ref)
        print("proj", n_, f"{e:.2e}", flush=True)
        assert e <= 2e-2, (n_, e)
    dh_ref = sum(g[n_][rows] @ wf[n_].T for n_ in ("wq", "wk", "wv"))
    e = rel(dh.cpu().double().numpy()[0][rows], dh_ref)
    print("dh", f"{e:.2e}", flush=True)
    assert e <= 2e-2, e
    got_w = {"wq": dwq.cpu().double().numpy(), "wk": dwk.cpu().double().numpy(), "wv": dwv.cpu().double().numpy()}
    for n_ in ("wq", "wk", "wv"):
        ms = rng.integers(0, dm, 24)
        ns = rng.integers(0, got_w[n_].shape[1], 24)
        ref = np.array([hf[:, m] @ g[n_][:, c] for m, c in zip(ms, ns)])
        scale = max(np.abs(ref).max(), 1e-30)
        e = float(np.abs(got_w[n_][ms, ns] - ref).max() / scale)
        print("dW", n_, f"{e:.2e}", flush=True)
        assert e <= 2e-2, (n_, e)
