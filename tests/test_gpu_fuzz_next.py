"""Randomized cases for the rows around the attention, through the C ABI, against the float64 oracle.

Streamed LM head (SFT): each case draws from a fixed seed the batch (1 or 2), the sequence length, d_model
(a multiple of 64), the vocabulary (a multiple of 64, up to 4096, or 8K-64K with shorter sequences so that
the loss kernels split each row into several vocabulary segments), the partition size ps (1 to the whole sequence), the
prompt length (positions that are not targets), the number of partitions per weight-gradient update, and
whether some labels fall outside the vocabulary (those positions are not targets either). Bars as the fixed
cases: loss to 1e-3 relative, row losses, dH and dW to 2e-2 of their largest magnitude.

Projections around the chunk attention: the batch, sequence length, chunk size (ragged last chunks included),
d_model, kv heads and group size, head size and storage type; the whole chunked layer (projections, chunk
forward, chunk backward, projection backward) against the dense oracle at 1e-5 (float32) / 2e-2 (bf16).

Stacks of attention layers with SpaCO's relay: the batch, sequence length, chunk size, number of layers, kv
heads and group size, head size, storage type, how many of the k chunks are drawn (t, with a drawn selection
seed; t = k with relay factor 1 is SeCO's exact backward) and the relay factor; the weight gradients of every
layer and dH_0 against the oracle's estimate at the same bars. bf16 rounding compounds with depth (each
layer's activations and gradients pass through bf16): a three-layer bf16 stack of 17 positions here reaches
1.7e-2 of the largest magnitude on its deepest weight gradients, against 2-6e-3 for one or two layers.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import lm_head as O
from oracle import projection as P
from sequence_chunked_exact_amd import workloads as W

import test_gpu_lm_head as TH
import test_gpu_proj as TP
import test_gpu_stack as TS
from oracle import selection
from oracle import stack as S

pytestmark = pytest.mark.gpu

N_HEAD, N_PROJ, N_STACK = 12, 12, 8


def draw_head(i):
    r = np.random.default_rng(5000 + i)
    B = int(r.integers(1, 3))
    wide = bool(r.random() < 0.35)  # 8K-64K vocabulary: the loss kernels split each row into 2-16 segments
    T = int(r.integers(1, 65 if wide else 301))
    dm = 64 * int(r.integers(1, 5))
    V = 64 * int(r.integers(128, 1025) if wide else r.integers(1, 65))
    ps = int(r.integers(1, T + 1))
    prompt = int(r.integers(0, T // 2 + 1))
    group = int(r.integers(1, 7))
    outside = bool(r.random() < 0.3)
    return B, T, dm, V, ps, prompt, group, outside


@pytest.mark.parametrize("i", range(N_HEAD))
def test_random_head_cases(i):
    B, T, dm, V, ps, prompt, group, outside = draw_head(i)
    print(f"[case head {i}] B={B} T={T} d_model={dm} vocab={V} ps={ps} prompt={prompt} dw_group={group} "
          f"outside={outside}", flush=True)
    wl = W.HeadWorkload(f"fuzz_head{i}", B, T, dm, V, ps, prompt, "bf16", seed=6000 + i)
    inp = W.make_head_inputs(wl)
    f = inp.f64
    labels = np.array(inp.raw["labels"], copy=True)
    if outside:  # a few target positions get labels past the vocabulary: not targets
        r = np.random.default_rng(7000 + i)
        pick = r.random(labels.shape) < 0.2
        labels[pick & (labels >= 0)] = V + 3
    ref_labels = np.where(labels >= V, -1, labels)  # the oracle's form: -1 for every non-target
    scale = O.target_scale(ref_labels)
    rl, dh, dw = TH.run_head(inp, ps, scale, labels_override=labels, dw_group=group)
    loss_ref, dh_ref, dw_ref = O.sft_streamed(f["h"], f["w"], ref_labels, ps, scale)
    rl_ref = O.row_losses(f["h"], f["w"], ref_labels)
    errs = {"row_loss": TH.rel(rl, rl_ref), "dh": TH.rel(dh, dh_ref), "dw": TH.rel(dw, dw_ref)}
    if loss_ref != 0.0:
        errs["loss"] = abs(scale * rl.sum() - loss_ref) / abs(loss_ref)
    print("          errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs.get("loss", 0.0) <= 1e-3
    for k in ("row_loss", "dh", "dw"):
        assert errs[k] <= 2e-2, (k, errs[k])


def draw_proj(i):
    r = np.random.default_rng(8000 + i)
    dtype = "f32" if r.random() < 0.25 else "bf16"
    B = int(r.integers(1, 3))
    T = int(r.integers(1, 701))
    C = int(r.integers(1, T + 1)) if r.random() < 0.6 else int(r.choice([64, 128, 256, 500]))
    C = max(1, min(C, T))
    dm = 64 * int(r.integers(1, 6))
    hkv = int(r.integers(1, 4))
    G = int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    return B, T, C, dm, hkv * G, hkv, d, dtype


@pytest.mark.parametrize("i", range(N_PROJ))
def test_random_projection_layers(i):
    B, T, C, dm, Hq, Hkv, d, dtype = draw_proj(i)
    print(f"[case proj {i}] B={B} T={T} C={C} d_model={dm} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
    wl = W.LayerWorkload(f"fuzz_proj{i}", B, T, C, dm, Hq, Hkv, d, dtype, seed=9000 + i)
    inp = W.make_layer_inputs(wl)
    got = TP.run_layer(wl, inp)
    f = inp.f64
    qr, kr, vr = P.qkv_forward(f["h"], f["wq"], f["wk"], f["wv"], Hq, Hkv)
    orf, _ = A.forward(qr, kr, vr, wl.softmax_scale)
    dwq, dwk, dwv, dh = P.layer_backward(f["h"], f["wq"], f["wk"], f["wv"], f["do"], Hq, Hkv, wl.softmax_scale)
    errs = {"q": TP.rel(got["q"], qr), "k": TP.rel(got["k"], kr), "v": TP.rel(got["v"], vr),
            "o": TP.rel(got["o"], orf), "dwq": TP.rel(got["dwq"], dwq), "dwk": TP.rel(got["dwk"], dwk),
            "dwv": TP.rel(got["dwv"], dwv), "dh": TP.rel(got["dh"], dh)}
    print("          errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    tol = 1e-5 if dtype == "f32" else 2e-2
    for n, e in errs.items():
        assert e <= tol, (n, e)


def draw_stack(i):
    r = np.random.default_rng(10000 + i)
    dtype = "f32" if r.random() < 0.3 else "bf16"
    B = int(r.integers(1, 3))
    T = int(r.integers(1, 321))
    C = max(1, min(T, int(r.integers(1, T + 1)) if r.random() < 0.6 else int(r.choice([32, 64, 128]))))
    L = int(r.integers(1, 4))
    hkv = int(r.integers(1, 3))
    G = int(r.integers(1, 3))
    d = int(r.choice([64, 128]))
    k = -(-T // C)
    t = int(r.integers(1, k + 1))
    seed = int(r.integers(0, 2**31))
    gamma = float(r.choice([1.0, 1.5, 2.0, k / t]))
    return B, T, C, L, hkv * G, hkv, d, dtype, t, seed, gamma


@pytest.mark.parametrize("i", range(N_STACK))
def test_random_stacks(i):
    B, T, C, L, Hq, Hkv, d, dtype, t, seed, gamma = draw_stack(i)
    print(f"[case stack {i}] B={B} T={T} C={C} layers={L} Hq={Hq} Hkv={Hkv} d={d} {dtype} t={t} seed={seed} "
          f"gamma={gamma:.3g}", flush=True)
    wl = W.StackWorkload(f"fuzz_stack{i}", B, T, C, L, Hq, Hkv, d, dtype, t, None, seed=11000 + i)
    inp = W.make_stack_inputs(wl)
    k = wl.n_chunks
    chunks = selection.select_chunks(k, t, seed)
    g = TS.GpuStack(wl, inp)
    g.forward()
    got = g.backward(chunks, gamma)
    args = TS.oracle_args(wl, inp)
    if len(chunks) == k and gamma == 1.0:
        ref = S.stack_dense_grad(*args)
    else:
        ref = S.spaco_estimate(*args, C, chunks, gamma)
    TS.compare(got, ref, 1e-5 if dtype == "f32" else 2e-2, f"          fuzz_stack{i}")
