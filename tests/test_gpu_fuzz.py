"""Randomized tile and tail cases, through the C ABI, against the float64 oracle.

Each case draws (from a fixed seed) the storage type, head size, kv heads and
group size, batch (1 or 2), sequence length, chunk size (ragged last chunks
included), a signed softmax scale, whether keys get the low-rank spike, which
dQ pass the backward takes, and one of three drivers: the whole-sequence
sweeps, per-chunk calls whose query-side tensors hold only the current chunk
(q_row_offset 0, q_capacity = the chunk's rows), or the sparse (SpaCO)
backward over t of the k chunks with a drawn t and selection seed. Every
element of O, LSE, dQ, dK and dV is compared at the parity bar: 1e-5
(float32) / 2e-2 (bf16), relative to the tensor's largest magnitude; LSE
relative to max(1, its largest magnitude), since float32 holds LSE to a relative
precision and the drawn scales and key spikes put it anywhere from 1 to ~20.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.selection import select_chunks
from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 40


def draw_case(i):
    r = np.random.default_rng(1000 + i)
    dtype = "f32" if r.random() < 0.3 else "bf16"
    d = int(r.choice([64, 128]))
    hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4]))
    batch = int(r.choice([1, 2]))
    T = int(r.integers(1, 1300))
    C = int(r.integers(1, T + 1)) if r.random() < 0.5 else int(r.choice([64, 128, 256, 500, 1024]))
    C = max(1, min(C, T))
    scale = float(r.choice([1.0, 1 / math.sqrt(d), 0.3])) * (-1.0 if r.random() < 0.25 else 1.0)
    spike = bool(r.random() < 0.4)
    ds = bool(r.random() < 0.5) and dtype == "bf16"
    mode = str(r.choice(["sweep", "per_chunk", "sparse"], p=[0.4, 0.3, 0.3]))
    k_chunks = -(-T // C)
    sparse = (int(r.integers(1, k_chunks + 1)), int(r.integers(0, 2**63))) if mode == "sparse" else None
    wl = W.Workload(f"fuzz{i}", batch, T, C, hkv * G, hkv, d, dtype, seed=2000 + i, softmax_scale=scale,
                    spike_rank=4 if spike else 0, spike_amp=3.0 if spike else 0.0)
    return wl, ds, mode, sparse


def run_case(wl, ds, mode, sparse):
    from sequence_chunked_exact_amd import binding as B
    inp = W.make_inputs(wl)
    t = {n: W.to_torch(inp.raw[n], DEV) for n in ("q", "k", "v", "do")}
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    T, sc = wl.seq_len, wl.softmax_scale
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    chunks = [wl.chunk_bounds(i) for i in range(wl.n_chunks)]
    sel = None
    if mode == "sweep":
        B.chunked_forward(q, k, v, o, lse, chunk=wl.chunk, softmax_scale=sc)
        B.chunked_backward(q, k, v, o, lse, do, dq, dk, dv, chunk=wl.chunk, softmax_scale=sc, ds_handover=ds)
    elif mode == "sparse":
        B.chunked_forward(q, k, v, o, lse, chunk=wl.chunk, softmax_scale=sc)
        sel = B.sparse_chunk_bwd(q, k, v, o, lse, do, dq, dk, dv, seq_len=T, chunk=wl.chunk, t=sparse[0],
                                 seed=sparse[1], softmax_scale=sc, ds_handover=ds)
    else:
        # query-side tensors of one chunk at a time: rows [s, s + c) copied out, computed, copied back
        # (clone, not contiguous(): a slice that is already contiguous would stay a view at an
        # offset the library's 16-byte alignment check rejects)
        for s, c in chunks:
            qc = q[:, :, s:s + c].clone()
            oc = torch.empty_like(qc)
            lc = torch.empty(qc.shape[:3], dtype=torch.float32, device=DEV)
            B.chunk_attn_fwd(qc, k, v, oc, lc, chunk_start=s, chunk_len=c, softmax_scale=sc)
            o[:, :, s:s + c] = oc
            lse[:, :, s:s + c] = lc
        for s, c in reversed(chunks):
            qc, oc, lc = (x[:, :, s:s + c].clone() for x in (q, o, lse))
            doc = do[:, :, s:s + c].clone()
            dqc = torch.empty(qc.shape, dtype=torch.float32, device=DEV)
            B.chunk_attn_bwd(qc, k, v, oc, lc, doc, dqc, dk, dv, chunk_start=s, chunk_len=c, softmax_scale=sc,
                             ds_handover=ds)
            dq[:, :, s:s + c] = dqc
    torch.cuda.synchronize()
    got = {"o": o.float(), "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    return inp, sel, {n: x.cpu().double().numpy() for n, x in got.items()}


def rel_inf(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_tiles_and_tails(i):
    wl, ds, mode, sparse = draw_case(i)
    print(f"[case {i}] B={wl.batch} T={wl.seq_len} C={wl.chunk} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
          f"d={wl.head_dim} {wl.dtype} scale={wl.softmax_scale:.3g} spike={wl.spike_rank > 0} ds={ds} "
          f"{mode}{'' if sparse is None else f' t={sparse[0]}/{wl.n_chunks} seed={sparse[1]}'}", flush=True)
    sys.stdout.flush()
    inp, sel, got = run_case(wl, ds, mode, sparse)
    f = inp.f64
    ro, rlse = A.forward(f["q"], f["k"], f["v"], wl.softmax_scale)
    if sel is None:
        rdq, rdk, rdv = A.backward(f["q"], f["k"], f["v"], f["do"], wl.softmax_scale)
    else:
        assert sel == select_chunks(wl.n_chunks, sparse[0], sparse[1])
        rdq, rdk, rdv = A.sparse_backward(f["q"], f["k"], f["v"], f["do"], wl.softmax_scale, wl.chunk, sel,
                                          wl.n_chunks)
    lse_err = float(np.abs(got["lse"] - rlse).max() / max(1.0, np.abs(rlse).max()))
    errs = {"o": rel_inf(got["o"], ro), "lse": lse_err,
            "dq": rel_inf(got["dq"], rdq), "dk": rel_inf(got["dk"], rdk), "dv": rel_inf(got["dv"], rdv)}
    print(f"          errors {errs}", flush=True)
    bar = 1e-5 if wl.dtype == "f32" else 2e-2
    for n, e in errs.items():
        assert e <= bar, (n, e)
