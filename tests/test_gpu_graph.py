"""The chunked attention step and the projection step inside a captured HIP
graph (torch.cuda.CUDAGraph): the library enqueues only kernels on the
caller's stream (zero fills are kernels, no memset nodes), so a captured step
replays to the same bits as the eager one. Each replay is compared with the
eager result, with eager work and synchronizations between the replays.
"""
import numpy as np
import pytest

from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_captured_chunked_step_replays_bitwise():
    import torch
    from sequence_chunked_exact_amd import binding as B
    wl = W.Workload("graph", 1, 640, 128, 8, 2, 128, "bf16", seed=43)
    print("[case] graph capture T=640 C=128", flush=True)
    inp = W.make_inputs(wl, keep_f64=False)
    dev = "cuda:0"
    q, k, v, do = (W.to_torch(inp.raw[n], dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=wl.chunk, softmax_scale=0.1)
    ws = torch.empty(max(B.chunk_attn_workspace_size(desc, B.CA_OP_SPARSE_BWD), 256), dtype=torch.uint8,
                     device=dev)

    def step():
        B.chunked_forward(q, k, v, o, lse, chunk=wl.chunk, softmax_scale=0.1)
        B.sparse_chunk_bwd(q, k, v, o, lse, do, dq, dk, dv, seq_len=wl.seq_len, chunk=wl.chunk, t=wl.n_chunks,
                           seed=0, softmax_scale=0.1, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (rep, name)
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_captured_projection_step_replays_bitwise():
    import torch
    from sequence_chunked_exact_amd import binding as B
    wl = W.LayerWorkload("graph_proj", 1, 512, 256, 512, 4, 2, 128, "bf16", seed=47)
    print("[case] graph capture projections", flush=True)
    inp = W.make_layer_inputs(wl, keep_f64=False)
    dev = "cuda:0"
    h, wq, wk, wv = (W.to_torch(inp.raw[n], dev) for n in ("h", "wq", "wk", "wv"))
    Bt, T, dm = h.shape
    q = torch.zeros(Bt, 4, T, 128, dtype=h.dtype, device=dev)
    k = torch.zeros(Bt, 2, T, 128, dtype=h.dtype, device=dev)
    v = torch.zeros_like(k)
    g = torch.randn(Bt, 4, T, 128, device=dev)
    gk, gv = torch.randn(Bt, 2, T, 128, device=dev), torch.randn(Bt, 2, T, 128, device=dev)
    dwq, dwk, dwv = (torch.zeros(dm, n * 128, device=dev) for n in (4, 2, 2))
    dh = torch.empty(Bt, T, dm, device=dev)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=wl.chunk)
    pws = torch.empty(max(B.qkv_proj_bwd_workspace_size(desc, dm), 256), dtype=torch.uint8, device=dev)

    def step():
        for t_ in (dwq, dwk, dwv):
            t_.zero_()
        for s in range(0, T, wl.chunk):
            B.qkv_proj_fwd(h, wq, wk, wv, q, k, v, chunk_start=s, chunk_len=wl.chunk, q_row_offset=s)
            B.qkv_proj_bwd(h, wq, wk, wv, q, k, g, gk, gv, dwq, dwk, dwv, dh, chunk_start=s, chunk_len=wl.chunk,
                           q_row_offset=s, workspace=pws)

    step()
    torch.cuda.synchronize()
    outs = (q, k, v, dwq, dwk, dwv, dh)
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan") if t.dtype == torch.float32 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), (rep, i)
        step()
        torch.cuda.synchronize()
    assert np.isfinite(dh.cpu().numpy()).all()
