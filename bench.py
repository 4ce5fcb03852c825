"""Benchmark: chunked exact causal attention forward + backward on one MI355X.

One step is one pass of the whole hot path over one sequence: the forward of
every chunk in ascending order (SeCO's inference-mode pass), then the backward
of every chunk in descending order into zeroed float32 dK/dV accumulators (for
the sparse workload: the t selected chunks, scaled by k/t). Inputs are resident
in HBM before timing starts. Prints one JSON line on stdout. The default run
(8b_layer, no --workload given) also measures the 4b_layer, 32b_layer and
sparse_64k workloads with fewer steps and reports them in the same line under
"other_workloads"; --no-others skips them, and --workload NAME measures that
workload alone.

FLOPs are causal only: 4*d per visible (query, key) pair and q head for the
forward (S and PV) and 10*d for the backward (S recompute, dP, dV, dQ, dK).

With --layer it measures instead the whole attention layer's chunked step on
an LLaMA3-8B-shaped layer: per chunk the QKV projections then the chunk
forward, then per chunk in descending order the chunk backward then the
projection backward (weight gradients and the input gradient). That mode
prints its own JSON line; its FLOPs add 2*d_model*(Hq+2*Hkv)*d per position
for each of the projection forward, the weight gradients and dH_in.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked causal attn fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
# The default run's line also carries these configurations of the same step.
OTHER_WORKLOADS = ("4b_layer", "32b_layer", "sparse_64k")
OTHER_STEPS, OTHER_WARMUP = 10, 2
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """The host the CPU baseline runs on: CPU model (from /proc/cpuinfo), the
    BLAS library numpy calls (threadpoolctl) and the threads it uses."""
    import numpy  # noqa: F401  (threadpoolctl lists only loaded libraries)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, " \
                   f"{i.get('architecture')} kernels)"
            threads = int(i.get("num_threads", threads))
    except Exception:
        pass
    return {"cores": threads, "cpu_model": model, "blas": blas}


def with_host(baseline):
    """Add the host description to a cpu_baseline record."""
    h = host_info()
    baseline.update({"cpu_model": h["cpu_model"], "blas": h["blas"]})
    return baseline



def timed_steps(B, torch, step, steps, pick_dominant, profile_steps=2):
    """Time `steps` calls of step() between two events on the current stream.

    Every launch the library brackets with events costs a little GPU time
    between kernels, so the per-kernel breakdown comes from `profile_steps`
    untimed steps with every kernel bracketed, and inside the timed region
    only the launches of the dominant kernel (pick_dominant(kernels)) carry
    events: its average duration is measured live over the timed region.
    Returns (ms_per_step, per_step_ms, kernels, dominant, (launches, total_ms)).
    """
    B.profile_select(None)
    B.profile_start()
    for _ in range(profile_steps):
        step()
    torch.cuda.synchronize()
    B.profile_stop()
    kernels = {n_: {"launches_per_step": c_ / profile_steps, "ms_per_step": t_ / profile_steps,
                    "avg_us": t_ / c_ * 1e3}
               for n_, (c_, t_) in B.profile_read().items() if c_}
    dom = pick_dominant(kernels)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    B.profile_select([dom])
    B.profile_start()
    e0.record(stream)
    for i in range(steps):
        step()
        marks[i].record(stream)
    torch.cuda.synchronize()
    B.profile_stop()
    B.profile_select(None)
    ms = e0.elapsed_time(marks[-1]) / steps
    per_step = [e0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, steps)]
    return ms, per_step, kernels, dom, B.profile_read()[dom]

def causal_pairs(start: int, length: int) -> int:
    """Visible (query, key) pairs of one chunk for one head."""
    return length * start + length * (length + 1) // 2


def flop_plan(wl, selected):
    d, hq = wl.head_dim, wl.n_q_heads
    chunks = [wl.chunk_bounds(i) for i in range(wl.n_chunks)]
    fwd_pairs = sum(causal_pairs(s, c) for s, c in chunks)
    bwd_chunks = selected if selected is not None else range(wl.n_chunks)
    bwd_pairs = sum(causal_pairs(*chunks[i]) for i in bwd_chunks)
    return {
        "fwd": 4 * d * hq * fwd_pairs,
        "bwd": 10 * d * hq * bwd_pairs,
        "dkdv": 8 * d * hq * bwd_pairs,     # S recompute, dP, dV, dK
        "bwd_pairs": bwd_pairs,
        "fwd_pairs": fwd_pairs,
    }


def cpu_baseline(wl, inp_raw, n_heads=8):
    """The float64 oracle on a bounded sample, extrapolated by causal FLOPs.

    Sample: the full causal forward + backward of the first `n_heads` query
    heads (each against its kv head) over the whole sequence.
    """
    import numpy as np
    from oracle import attention as A
    from sequence_chunked_exact_amd import workloads as W
    threads = host_info()["cores"]
    G = wl.n_q_heads // wl.n_kv_heads

    def head(name, h):
        a = inp_raw[name][:, h:h + 1]
        return W.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    t0 = time.perf_counter()
    for h in range(n_heads):
        q, do = head("q", h), head("do", h)
        k, v = head("k", h // G), head("v", h // G)
        A.forward(q, k, v, wl.softmax_scale)
        A.backward(q, k, v, do, wl.softmax_scale)
    dt = time.perf_counter() - t0
    pairs = wl.seq_len * (wl.seq_len + 1) // 2
    sample_flops = 14 * wl.head_dim * pairs * n_heads
    rate = sample_flops / dt
    plan = flop_plan(wl, None)
    total = plan["fwd"] + plan["bwd"]
    tokens_per_s = wl.seq_len * rate / total
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle forward+backward of query heads 0..{n_heads - 1} of "
                      f"{wl.n_q_heads} over all {wl.seq_len} positions ({dt:.1f} s, "
                      f"{rate / 1e9:.1f} GFLOP/s), extrapolated to all heads by causal FLOPs",
            "seconds": dt, "gflops": rate / 1e9}


def layer_cpu_baseline(wl, raw, rows=2048, n_heads=8):
    """The float64 oracle on a bounded sample of the layer step, extrapolated by FLOPs:
    the projections' forward and backward over the first `rows` positions, and the
    attention forward + backward of `n_heads` query heads over all positions."""
    import numpy as np
    from oracle import attention as A
    from oracle import projection as P
    from sequence_chunked_exact_amd import workloads as W
    threads = host_info()["cores"]
    f = {n: (W.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)) for n, a in raw.items()}
    Hq, Hkv, d, dm, T = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_model, wl.seq_len
    G = Hq // Hkv
    t0 = time.perf_counter()
    h = f["h"][:, :rows]
    q, k, v = P.qkv_forward(h, f["wq"], f["wk"], f["wv"], Hq, Hkv)
    P.qkv_backward(h, f["wq"], f["wk"], f["wv"], q, k, v)
    t_proj = time.perf_counter() - t0
    t_attn = 0.0
    for hh in range(n_heads):
        kv = hh // G
        qh, kh, vh = P.qkv_forward(f["h"][:1], f["wq"][:, hh * d:(hh + 1) * d], f["wk"][:, kv * d:(kv + 1) * d],
                                   f["wv"][:, kv * d:(kv + 1) * d], 1, 1)
        t1 = time.perf_counter()
        A.forward(qh, kh, vh, wl.softmax_scale)
        A.backward(qh, kh, vh, f["do"][:1, hh:hh + 1], wl.softmax_scale)
        t_attn += time.perf_counter() - t1
    proj_rate = 3 * 2 * rows * dm * (Hq + 2 * Hkv) * d / t_proj
    pairs = T * (T + 1) // 2
    attn_rate = 14 * d * pairs * n_heads / t_attn
    Bt = f["h"].shape[0]
    total_s = Bt * (3 * 2 * T * dm * (Hq + 2 * Hkv) * d / proj_rate + 14 * d * pairs * Hq / attn_rate)
    return {"value": Bt * T / total_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle: projections forward+backward over the first {rows} of {T} positions "
                      f"({t_proj:.1f} s) and attention forward+backward of {n_heads} of {Hq} query heads over "
                      f"all positions ({t_attn:.1f} s), each extrapolated to the whole layer by FLOPs",
            "seconds": t_proj + t_attn}


def layer_main(args):
    import numpy as np
    import torch
    from sequence_chunked_exact_amd import binding as B
    from sequence_chunked_exact_amd import workloads as W

    wl = W.LAYER_WORKLOADS["8b_attn_layer"]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name} inputs")
    inp = W.make_layer_inputs(wl, keep_f64=False)
    h, wq, wk, wv, do = (W.to_torch(inp.raw[n], dev) for n in ("h", "wq", "wk", "wv", "do"))
    Bt, T, dm = h.shape
    Hq, Hkv, d, C = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk
    sc = wl.softmax_scale
    f32 = torch.float32
    q = torch.zeros(Bt, Hq, T, d, dtype=h.dtype, device=dev)
    k = torch.zeros(Bt, Hkv, T, d, dtype=h.dtype, device=dev)
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(Bt, Hq, T, dtype=f32, device=dev)
    dq = torch.zeros(Bt, Hq, T, d, dtype=f32, device=dev)
    dk = torch.zeros(Bt, Hkv, T, d, dtype=f32, device=dev)
    dv = torch.zeros_like(dk)
    dwq = torch.zeros(dm, Hq * d, dtype=f32, device=dev)
    dwk = torch.zeros(dm, Hkv * d, dtype=f32, device=dev)
    dwv = torch.zeros_like(dwk)
    dh = torch.empty(Bt, T, dm, dtype=f32, device=dev)
    starts = list(range(0, T, C))
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=C)
    ws = torch.empty(max(B.chunk_attn_workspace_size(desc, B.CA_OP_BWD), 256), dtype=torch.uint8, device=dev)
    # bf16 layers: the weights' transpose is written once per backward sweep (qkv_proj_weights_t),
    # so each chunk's projection backward needs only the gradient part of its workspace
    wt_bytes = B.qkv_proj_weights_t_bytes(desc, dm)
    wcat_t = torch.empty(max(wt_bytes, 16), dtype=torch.uint8, device=dev) if wt_bytes else None
    pws = torch.empty(max(B.qkv_proj_bwd_workspace_size(desc, dm) - wt_bytes, 256), dtype=torch.uint8, device=dev)

    def step():
        for s in starts:
            c = min(C, T - s)
            B.qkv_proj_fwd(h, wq, wk, wv, q, k, v, chunk_start=s, chunk_len=c, q_row_offset=s)
            B.chunk_attn_fwd(q, k, v, o, lse, chunk_start=s, chunk_len=c, q_row_offset=s, softmax_scale=sc)
        for t_ in (dk, dv, dwq, dwk, dwv):
            t_.zero_()
        if wcat_t is not None:
            B.qkv_proj_weights_t(wq, wk, wv, q, k, out=wcat_t)
        for s in reversed(starts):
            c = min(C, T - s)
            B.chunk_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, chunk_start=s, chunk_len=c, q_row_offset=s,
                             softmax_scale=sc, workspace=ws)
            B.qkv_proj_bwd(h, wq, wk, wv, q, k, dq, dk, dv, dwq, dwk, dwv, dh, chunk_start=s, chunk_len=c,
                           q_row_offset=s, workspace=pws, w_cat_t=wcat_t)

    log(f"[bench] layer warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} layer steps")
    pairs = sum(causal_pairs(s, min(C, T - s)) for s in starts)
    attn_flops = 14 * d * Hq * pairs
    proj_flops = 3 * 2 * Bt * T * dm * (Hq + 2 * Hkv) * d
    total = attn_flops + proj_flops
    # algorithmic FLOPs of the products each kernel carries (as in the attention step)
    kflops = {"proj": proj_flops, "fwd": 4 * d * Hq * pairs, "dkdv": 8 * d * Hq * pairs, "dq": 2 * d * Hq * pairs,
              "bwd": 10 * d * Hq * pairs}
    ms, _, kernels, dom, (n_dom, t_dom) = timed_steps(
        B, torch, step, args.steps,
        lambda k_: max((n_ for n_ in k_ if n_ in kflops), key=lambda n_: k_[n_]["ms_per_step"]))
    log(f"[bench] {ms:.3f} ms/layer step; kernels " + json.dumps(kernels))
    from sequence_chunked_exact_amd.profile_summary import read_traffic
    dom_per_launch = kflops[dom] / (n_dom / args.steps)
    dom_achieved = dom_per_launch / (t_dom / n_dom * 1e-3) / 1e12
    out = {
        "metric": "chunked attention layer (QKV projections + causal attn) fwd+bwd tokens/s, 1 GPU",
        "value": Bt * T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "tflops": total / (ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "config": {"workload": wl.name, "batch": Bt, "seq_len": T, "chunk": C, "d_model": dm, "n_q_heads": Hq,
                   "n_kv_heads": Hkv, "head_dim": d, "softmax_scale": sc, "flops_per_step": total,
                   "projection_flops_per_step": proj_flops},
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": dom_achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom_achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(os.path.join(ROOT, "profiles", f"{dom}_{wl.name}.md"), dom),
                     "avg_launch_us": t_dom / n_dom * 1e3, "flops_per_launch": dom_per_launch},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = with_host(layer_cpu_baseline(wl, inp.raw))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def stack_flops(wl, T, drawn):
    """FLOPs of one SpaCO step on a layer stack, by kernel: the inference-mode pass
    over every chunk and layer, then per drawn chunk the rebuild (projections and
    attention forward) and the backward (attention and projections)."""
    Hq, Hkv, d, dm, C, L = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_model, wl.chunk, wl.n_layers
    proj_row = 2 * dm * (Hq + 2 * Hkv) * d          # one row of Q|K|V
    f = {"proj": 0, "fwd": 0, "bwd": 0}
    for s in range(0, T, C):
        c = min(C, T - s)
        f["proj"] += L * c * proj_row
        f["fwd"] += L * 4 * d * causal_pairs(s, c) * Hq
    for j in drawn:
        s = j * C
        c = min(C, T - s)
        pairs = causal_pairs(s, c)
        f["proj"] += L * c * proj_row * 3           # rebuild, dW, dH
        f["fwd"] += L * 4 * d * pairs * Hq          # rebuild
        f["bwd"] += L * 10 * d * pairs * Hq        # dK/dV (8 d) and dQ (2 d), one launch
    return f


def stack_cpu_baseline(wl, raw, sample_len=4096):
    """The float64 stack oracle (oracle.stack.spaco_estimate) on the workload cut to its
    first `sample_len` positions with the last chunk drawn, its rate in the GPU path's
    FLOP accounting extrapolated to the full step."""
    import numpy as np
    from oracle import stack as S
    from sequence_chunked_exact_amd import workloads as W
    threads = host_info()["cores"]

    def f64(a):
        return W.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    Ts = min(sample_len, wl.seq_len)
    h0 = f64(raw["h0"][:, :Ts])
    dy = f64(raw["dy"][:, :Ts])
    weights = [(f64(raw[f"wq{l}"]), f64(raw[f"wk{l}"]), f64(raw[f"wv{l}"])) for l in range(wl.n_layers)]
    last = (Ts - 1) // wl.chunk
    t0 = time.perf_counter()
    S.spaco_estimate(h0, weights, dy, wl.n_q_heads, wl.n_kv_heads, wl.softmax_scale, wl.chunk, [last],
                     wl.relay_factor)
    dt = time.perf_counter() - t0
    rate = sum(stack_flops(wl, Ts, [last]).values()) / dt
    return rate, dt, threads


def stack_main(args):
    import numpy as np
    import torch
    from sequence_chunked_exact_amd import binding as B
    from sequence_chunked_exact_amd import workloads as W

    wl = W.STACK_WORKLOADS["8b_stack4_spaco"]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name} inputs")
    inp = W.make_stack_inputs(wl, keep_f64=False)
    r = inp.raw
    h0, dy = W.to_torch(r["h0"], dev), W.to_torch(r["dy"], dev)
    Bt, T, dm = h0.shape
    Hq, Hkv, d, C, L = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk, wl.n_layers
    f32 = torch.float32
    layers = []
    for l in range(L):
        layers.append({"wq": W.to_torch(r[f"wq{l}"], dev), "wk": W.to_torch(r[f"wk{l}"], dev),
                       "wv": W.to_torch(r[f"wv{l}"], dev),
                       "k_cache": torch.zeros(Bt, Hkv, T, d, dtype=h0.dtype, device=dev),
                       "v_cache": torch.zeros(Bt, Hkv, T, d, dtype=h0.dtype, device=dev),
                       "dk_acc": torch.empty(Bt, Hkv, T, d, dtype=f32, device=dev),
                       "dv_acc": torch.empty(Bt, Hkv, T, d, dtype=f32, device=dev),
                       "dwq": torch.zeros(dm, Hq * d, dtype=f32, device=dev),
                       "dwk": torch.zeros(dm, Hkv * d, dtype=f32, device=dev),
                       "dwv": torch.zeros(dm, Hkv * d, dtype=f32, device=dev)})
    dh0 = torch.zeros(Bt, T, dm, dtype=f32, device=dev)
    desc = B.stack_desc(h0, layers, chunk=C, softmax_scale=wl.softmax_scale)
    ws = B.spaco_stack_workspace(desc, L, h0)
    k = wl.n_chunks
    drawn = B.chunk_select(k, wl.t, args.seed)
    gamma = wl.relay_factor

    def step():
        for lay in layers:
            for n_ in ("dwq", "dwk", "dwv"):
                lay[n_].zero_()
        B.spaco_stack_forward(h0, layers, chunk=C, softmax_scale=wl.softmax_scale, workspace=ws)
        B.spaco_stack_backward(h0, dy, dh0, layers, chunk=C, chunks=drawn, relay_factor=gamma,
                               softmax_scale=wl.softmax_scale, workspace=ws)

    log(f"[bench] stack warmup {args.warmup}; drawn chunks {drawn}, relay factor {gamma}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} stack steps")
    kflops = stack_flops(wl, T, drawn)
    total = sum(kflops.values())
    ms, _, kernels, dom, (n_l, t_l) = timed_steps(
        B, torch, step, args.steps,
        lambda k_: max((n_ for n_ in k_ if n_ in kflops), key=lambda n_: k_[n_]["ms_per_step"]))
    log(f"[bench] {ms:.3f} ms/stack step; kernels " + json.dumps(kernels))
    per_launch = kflops[dom] / (n_l / args.steps)
    achieved = per_launch / (t_l / n_l * 1e-3) / 1e12
    from sequence_chunked_exact_amd.profile_summary import read_traffic
    out = {
        "metric": "SpaCO step on an attention-layer stack (inference pass + relayed backward of t drawn chunks) "
                  "tokens/s, 1 GPU",
        "value": Bt * T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "tflops": total / (ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "config": {"workload": wl.name, "batch": Bt, "seq_len": T, "chunk": C, "n_layers": L, "d_model": dm,
                   "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "t": wl.t, "k": k, "drawn": drawn,
                   "relay_factor": gamma, "flops_per_step": total, "flops_by_kernel": kflops},
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(os.path.join(ROOT, "profiles", f"{dom}_{wl.name}.md"), dom),
                     "avg_launch_us": t_l / n_l * 1e3, "flops_per_launch": per_launch},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        rate, dt, threads = stack_cpu_baseline(wl, r)
        out["cpu_baseline"] = with_host({"value": Bt * T / (total / rate), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"float64 stack oracle on the first 4096 positions with the last chunk "
                                         f"drawn ({dt:.1f} s, {rate / 1e9:.1f} GFLOP/s in this step's FLOP "
                                         f"accounting), extrapolated to the full step by FLOPs",
                               "seconds": dt})
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def head_bytes(T, dm, V, ps, group, B=1):
    """Algorithmic HBM bytes of the head's three products over one step: per
    partition of r positions, the logits product reads W^T and H rows and writes
    the float32 logits; dH reads dZ (bf16) and W and writes its split-k partials
    (16 splits for the LLaMA3 vocabulary: the largest count up to 16 whose parts of
    whole 64-wide vocabulary slices are all non-empty); per group of partitions, dW reads dZ
    and H rows and reads + writes the float32 weight gradient. At these sizes
    (about 125 FLOP per byte, under MI355X's ~310 FLOP/B balance of bf16 MFMA to
    HBM) the head is bound by memory."""
    wbytes = V * dm * 2
    n = V // 64
    splits = next((s for s in range(16, 1, -1) if (s - 1) * ((n + s - 1) // s) < n), 1)
    total = 0
    for s0 in range(0, T, ps):
        r = min(ps, T - s0)
        total += wbytes + B * r * dm * 2 + B * r * V * 4            # logits
        total += B * r * V * 2 + wbytes + splits * r * dm * 4       # dH partials
    for g0 in range(0, T, ps * group):
        rows = min(ps * group, T - g0)
        total += B * rows * V * 2 + B * rows * dm * 2 + 2 * V * dm * 4  # dW
    return total


def head_main(args):
    import numpy as np
    import torch
    from sequence_chunked_exact_amd import binding as B
    from sequence_chunked_exact_amd import workloads as W

    wl = W.HEAD_WORKLOADS["8b_head_sft"]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name} inputs")
    inp = W.make_head_inputs(wl, keep_f64=False)
    h = W.to_torch(inp.raw["h"], dev)
    w = W.to_torch(inp.raw["w"], dev)
    lab_np = inp.raw["labels"]
    labels = torch.from_numpy(np.ascontiguousarray(lab_np)).to(dev)
    Bt, T, dm = h.shape
    V = w.shape[0]
    scale = 1.0 / float((lab_np >= 0).sum())
    wt = torch.empty(dm, V, dtype=h.dtype, device=dev)
    row_loss = torch.empty(Bt, T, device=dev)
    dh = torch.empty(Bt, T, dm, device=dev)
    dw = torch.zeros(V, dm, device=dev)
    ws = B.lm_head_sweep_workspace(h, w, wl.ps, wl.dw_group)

    def step():
        dw.zero_()
        B.lm_head_transpose(w, wt)
        B.lm_head_sft(h, w, wt, labels, row_loss, dh, dw, loss_scale=scale, ps=wl.ps, dw_group=wl.dw_group,
                      workspace=ws)

    log(f"[bench] head warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} head steps")
    ms, _, kernels, _, (n_h, t_h) = timed_steps(B, torch, step, args.steps, lambda k_: "head")
    flops = 3 * 2 * Bt * T * V * dm                     # logits, dH, dW
    log(f"[bench] {ms:.3f} ms/head step; kernels " + json.dumps(kernels))
    per_launch = flops / (n_h / args.steps)
    achieved = per_launch / (t_h / n_h * 1e-3) / 1e12
    hbytes = head_bytes(T, dm, V, wl.ps, wl.dw_group, Bt)
    bytes_per_launch = hbytes / (n_h / args.steps)
    achieved_gbs = bytes_per_launch / (t_h / n_h * 1e-3) / 1e9
    loss = scale * float(row_loss.sum().item())
    from sequence_chunked_exact_amd.profile_summary import read_traffic
    out = {
        "metric": "streamed LM head SFT loss + gradients (ps_head partitions) tokens/s, 1 GPU",
        "value": Bt * T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "tflops": flops / (ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "config": {"workload": wl.name, "batch": Bt, "seq_len": T, "d_model": dm, "vocab": V, "ps_head": wl.ps,
                   "dw_group": wl.dw_group, "prompt": wl.prompt, "flops_per_step": flops, "loss": loss},
        "kernels": kernels,
        "roofline": {"kernel": "head", "bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / PEAK_HBM_GBS,
                     "traffic": read_traffic(os.path.join(ROOT, "profiles", f"head_{wl.name}.md"), "head"),
                     "avg_launch_us": t_h / n_h * 1e3, "bytes_per_launch": bytes_per_launch,
                     "flops_per_launch": per_launch, "mfma_tflops": achieved,
                     "mfma_frac": achieved / PEAK_BF16_TFLOPS},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        from oracle import lm_head as O
        threads = host_info()["cores"]
        hf = W.bf16_bits_to_f64(inp.raw["h"])
        wf = W.bf16_bits_to_f64(inp.raw["w"])
        n_part = 20
        t0 = time.perf_counter()
        for i in range(n_part):
            s0 = wl.prompt + i * wl.ps
            O.sft_partition(hf, wf, lab_np, slice(s0, s0 + wl.ps), scale)
        dt = time.perf_counter() - t0
        rate = 3 * 2 * n_part * wl.ps * V * dm / dt
        out["cpu_baseline"] = with_host({"value": Bt * T / (flops / rate), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"float64 oracle on {n_part} partitions of {wl.ps} positions at the full "
                                         f"vocabulary ({dt:.1f} s, {rate / 1e9:.1f} GFLOP/s), extrapolated to all "
                                         f"{T} positions by FLOPs", "seconds": dt})
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="measure this workload only (default: 8b_layer, plus the other workloads in the same line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layer", action="store_true",
                    help="measure the whole attention layer step (QKV projections + attention)")
    ap.add_argument("--stack", action="store_true",
                    help="measure SpaCO's step on a stack of attention layers (relayed cache gradients)")
    ap.add_argument("--seed", type=int, default=0, help="chunk draw seed for --stack")
    ap.add_argument("--head", action="store_true", help="measure the streamed LM head (SFT) step")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads that the default 8b_layer run also measures")
    ap.add_argument("--ds-handover", action="store_true",
                    help="give the backward the CA_OP_BWD_DS workspace (dS handed to the dQ pass; memory grows "
                         "with the sequence) instead of the bounded one")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.layer:
        return layer_main(args)
    if args.stack:
        return stack_main(args)
    if args.head:
        return head_main(args)

    import torch

    from sequence_chunked_exact_amd import workloads as W

    wl = W.WORKLOADS[args.workload or "8b_layer"]
    out, inp = measure_attention(wl, args.steps, args.warmup, args.ds_handover)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = with_host(cpu_baseline(wl, inp.raw))
    else:
        out["cpu_baseline"] = None
    del inp
    # The other configurations of the same step, measured in the same run
    # with fewer steps (the line's value stays the one workload's).
    if not args.no_others and args.workload is None and not args.ds_handover:
        others = {}
        for name in OTHER_WORKLOADS:
            torch.cuda.empty_cache()
            o, _ = measure_attention(W.WORKLOADS[name], OTHER_STEPS, OTHER_WARMUP, False)
            others[name] = {k_: o[k_] for k_ in ("value", "unit", "steps", "warmup", "ms_per_step", "tflops",
                                                  "pct_bf16_peak", "tflops_fwd", "tflops_bwd", "kernels")}
            others[name]["config"] = o["config"]
            others[name]["roofline"] = {k_: o["roofline"].get(k_) for k_ in ("kernel", "frac", "achieved",
                                                                            "avg_launch_us", "traffic")}
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


def measure_attention(wl, steps, warmup, ds_handover):
    """One workload's attention step (every chunk's forward, then the backward
    of every chunk or of the drawn ones): the bench line without the CPU
    baseline, and the inputs."""
    import numpy as np
    import torch
    from sequence_chunked_exact_amd import binding as B
    from sequence_chunked_exact_amd import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name} inputs")
    inp = W.make_inputs(wl, keep_f64=False)
    q, k, v, do = (W.to_torch(inp.raw[n], dev) for n in ("q", "k", "v", "do"))
    T, C = wl.seq_len, wl.chunk
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    desc = B.make_desc(q, k, chunk_start=0, chunk_len=C, softmax_scale=wl.softmax_scale)
    # The backward's workspace: the bounded one (the chunk's row statistics; the
    # dQ pass recomputes dS), or with --ds-handover room for dS^T of a chunk
    # against the whole prefix (memory that grows with the sequence).
    ws_op = B.CA_OP_BWD_DS if ds_handover else B.CA_OP_SPARSE_BWD
    ws_bytes = B.chunk_attn_workspace_size(desc, ws_op)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    sparse = wl.sparse_t > 0
    t_sel = wl.sparse_t if sparse else wl.n_chunks      # t = k: every chunk, scale 1
    seed = wl.select_seed

    def step():
        B.chunked_forward(q, k, v, o, lse, chunk=C, softmax_scale=wl.softmax_scale)
        return B.sparse_chunk_bwd(q, k, v, o, lse, do, dq, dk, dv, seq_len=T, chunk=C, t=t_sel, seed=seed,
                                  softmax_scale=wl.softmax_scale, workspace=ws)

    log(f"[bench] {wl.name}: warmup {warmup}")
    for _ in range(warmup):
        selected = step()
    torch.cuda.synchronize()

    log(f"[bench] {wl.name}: timing {steps} steps")
    sel = {}

    def run():
        sel["v"] = step()

    # roofline for the kernel with the most GPU time; its algorithmic FLOPs are
    # the products it carries (forward: S, PV = 4d per pair; dK/dV: S, dP, dV,
    # dK = 8d per pair; dQ: the dQ product, 2d; the fused backward launch, dK/dV
    # and dQ together: 10d; recomputed products are not counted)
    t_wall = time.perf_counter()
    ms, per_step, kernels, dom, (n_launch, tot_ms) = timed_steps(
        B, torch, run, steps, lambda k_: max(k_, key=lambda n_: k_[n_]["ms_per_step"]))
    wall = time.perf_counter() - t_wall
    selected = sel["v"]
    log(f"[bench] {wl.name}: {ms:.3f} ms/step (wall incl. the profiled steps {wall / (steps + 2) * 1e3:.3f} "
        "ms/step)")
    log("[bench] kernels " + json.dumps(kernels))

    plan = flop_plan(wl, selected if sparse else None)
    total_flops = plan["fwd"] + plan["bwd"]
    tflops = total_flops / (ms * 1e-3) / 1e12
    dom_flops = {"fwd": plan["fwd"], "dkdv": plan["dkdv"], "dq": plan["bwd"] // 5, "bwd": plan["bwd"]}.get(dom)
    roof = {"kernel": dom, "bound": "mfma", "achieved": None, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": None, "traffic": None}
    if dom_flops is not None:
        per_launch_flops = dom_flops / (n_launch / steps)
        avg_s = tot_ms / n_launch * 1e-3
        achieved = per_launch_flops / avg_s / 1e12
        roof.update({"achieved": achieved, "frac": achieved / PEAK_BF16_TFLOPS,
                     "avg_launch_us": avg_s * 1e6, "flops_per_launch": per_launch_flops})
    from sequence_chunked_exact_amd.profile_summary import read_traffic
    roof["traffic"] = read_traffic(os.path.join(ROOT, "profiles", f"{dom}_{wl.name}.md"), dom)
    fwd_ms = kernels.get("fwd", {}).get("ms_per_step", 0.0)
    bwd_ms = sum(kernels.get(k_, {}).get("ms_per_step", 0.0) for k_ in ("delta", "dkdv", "dq", "bwd", "zero"))

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(min(per_step)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "tflops_fwd": plan["fwd"] / (fwd_ms * 1e-3) / 1e12 if fwd_ms else None,
        "tflops_bwd": plan["bwd"] / (bwd_ms * 1e-3) / 1e12 if bwd_ms else None,
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": T, "chunk": C,
                   "n_chunks": wl.n_chunks, "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "softmax_scale": wl.softmax_scale,
                   "key_spike": (f"rank {wl.spike_rank} amplitude {wl.spike_amp}" if wl.spike_rank else None),
                   "sparse_t": wl.sparse_t or None, "selected_chunks": selected if sparse else None,
                   "causal_flops_per_step": total_flops, "workspace_bytes": ws_bytes,
                   "dq_pass": "stored dS (CA_OP_BWD_DS)" if ds_handover else "recompute (CA_OP_SPARSE_BWD)"},
        "kernels": kernels,
        "roofline": roof,
    }
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return out, inp


if __name__ == "__main__":
    main()
