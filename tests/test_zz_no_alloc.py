"""chunk_attn_bwd_noalloc (the backward that takes its scratch from a static
device array instead of a workspace) against chunk_attn_bwd with its minimal
workspace, through the C ABI: two sweeps in a row, the second on a smaller
input, each compared bitwise with the workspace path (the same kernels) and
with the float64 oracle at the parity bar."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def sweep(B, wl, inp, noalloc):
    t = {n: W.to_torch(inp.raw[n], DEV) for n in ("q", "k", "v", "do")}
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    T, C, sc = wl.seq_len, wl.chunk, wl.softmax_scale
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.chunked_forward(q, k, v, o, lse, chunk=C, softmax_scale=sc)
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=C, softmax_scale=sc)
    ws = torch.empty(max(B.chunk_attn_workspace_size(desc, B.CA_OP_BWD_MIN), 256), dtype=torch.uint8, device=DEV)
    for i in reversed(range(wl.n_chunks)):
        s, c = wl.chunk_bounds(i)
        kw = dict(chunk_start=s, chunk_len=c, q_row_offset=s, softmax_scale=sc)
        if noalloc:
            B.chunk_attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, **kw)
        else:
            B.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    return {n: x.cpu().double().numpy() for n, x in (("dq", dq), ("dk", dk), ("dv", dv))}


def rel_inf(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def test_noalloc_backward_equals_workspace_backward_two_calls():
    from sequence_chunked_exact_amd import binding as B
    cases = [
        W.Workload("noalloc_a", 1, 1500, 512, 8, 2, 128, "bf16", seed=71, spike_rank=4, spike_amp=3.0),
        W.Workload("noalloc_b", 1, 300, 96, 4, 2, 64, "f32", seed=72, softmax_scale=0.125),   # smaller
    ]
    for wl in cases:
        inp = W.make_inputs(wl)
        print(f"[case] {wl.name} T={wl.seq_len} C={wl.chunk} {wl.dtype}", flush=True)
        got = sweep(B, wl, inp, noalloc=True)
        ref_ws = sweep(B, wl, inp, noalloc=False)
        for n in got:
            assert np.array_equal(got[n], ref_ws[n]), n
        f = inp.f64
        rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], wl.softmax_scale)
        bar = 1e-5 if wl.dtype == "f32" else 2e-2
        errs = {n: rel_inf(got[n], r) for n, r in (("dq", rdq), ("dk", rdk), ("dv", rdv))}
        print(f"       errors {errs}", flush=True)
        for n, e in errs.items():
            assert e <= bar, (n, e)


def test_noalloc_rejects_rows_beyond_the_scratch():
    from sequence_chunked_exact_amd import binding as B
    q = torch.zeros(1, 64, 32768, 64, dtype=torch.bfloat16, device=DEV)     # 64 * 32768 rows > ~1M
    k = torch.zeros(1, 8, 32768, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 64, 32768, device=DEV)
    f = torch.zeros(1, 64, 32768, 64, device=DEV)
    fk = torch.zeros(1, 8, 32768, 64, device=DEV)
    with pytest.raises(B.ChunkAttnError) as ei:
        B.chunk_attn_bwd_noalloc(q, k, k, q, lse, q, f, fk, fk, chunk_start=0, chunk_len=32768)
    assert ei.value.code == -5
