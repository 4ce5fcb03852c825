"""GPU parity of the streamed LM head under SFT (lm_head_transpose /
lm_head_sft_partition through the C ABI) against the float64 oracle
(oracle.lm_head). bf16 storage only; bar 2e-2 per tensor (max error over max
reference magnitude), loss to 1e-3 relative.
"""
import numpy as np
import pytest

from oracle import lm_head as O
from sequence_chunked_exact_amd import workloads as W

pytestmark = pytest.mark.gpu


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-30))


def run_head(inp, ps, scale, labels_override=None, dw_group=1):
    import torch
    from sequence_chunked_exact_amd import binding as Bn
    dev = "cuda:0"
    h = W.to_torch(inp.raw["h"], dev)
    w = W.to_torch(inp.raw["w"], dev)
    lab = inp.raw["labels"] if labels_override is None else labels_override
    labels = torch.from_numpy(np.ascontiguousarray(lab)).to(dev)
    B, T, dm = h.shape
    V = w.shape[0]
    wt = torch.empty(dm, V, dtype=h.dtype, device=dev)
    row_loss = torch.full((B, T), float("nan"), device=dev)
    dh = torch.full((B, T, dm), float("nan"), device=dev)
    dw = torch.zeros(V, dm, device=dev)
    Bn.lm_head_transpose(w, wt)
    Bn.lm_head_sft(h, w, wt, labels, row_loss, dh, dw, loss_scale=scale, ps=ps, dw_group=dw_group)
    torch.cuda.synchronize()
    return row_loss.cpu().double().numpy(), dh.cpu().double().numpy(), dw.cpu().double().numpy()


CASES = [
    # name, B, T, d_model, vocab, ps, prompt, dw_group (partitions per weight-gradient update)
    ("ragged_partitions", 1, 250, 256, 1024, 100, 20, 1),
    ("batch2_ps64", 2, 128, 128, 2048, 64, 0, 1),
    ("ps1_tiny_vocab", 1, 9, 64, 64, 1, 3, 1),
    ("one_partition_all_rows", 2, 70, 192, 448, 100, 5, 1),
    ("grouped_dw_short_last_group", 1, 250, 256, 1024, 40, 10, 3),
    ("grouped_dw_batch2_group_exceeds_sequence", 2, 130, 128, 512, 32, 0, 8),
    # 17 vocabulary slices of 64: dH splits into 9 parts of 2 slices, the last of 1 (the GEMM's
    # shorter last split-k entry)
    ("uneven_split_vocab_1088", 1, 120, 128, 1088, 50, 4, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_head_parity(case):
    name, B, T, dm, V, ps, prompt, group = case
    print(f"[case] {name}", flush=True)
    wl = W.HeadWorkload(name, B, T, dm, V, ps, prompt, "bf16", seed=29)
    inp = W.make_head_inputs(wl)
    f = inp.f64
    scale = O.target_scale(f["labels"])
    rl, dh, dw = run_head(inp, ps, scale, dw_group=group)
    loss_ref, dh_ref, dw_ref = O.sft_streamed(f["h"], f["w"], f["labels"], ps, scale)
    rl_ref = O.row_losses(f["h"], f["w"], f["labels"])
    loss = scale * rl.sum()
    errs = {"loss": abs(loss - loss_ref) / abs(loss_ref), "row_loss": rel(rl, rl_ref), "dh": rel(dh, dh_ref),
            "dw": rel(dw, dw_ref)}
    print(name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] <= 1e-3
    for k in ("row_loss", "dh", "dw"):
        assert errs[k] <= 2e-2, (k, errs[k])
    assert np.all(rl[:, :prompt] == 0.0)


def test_labels_outside_the_vocabulary_are_not_targets():
    wl = W.HeadWorkload("oob_labels", 1, 64, 128, 256, 32, 0, "bf16", seed=31)
    inp = W.make_head_inputs(wl)
    lab = inp.raw["labels"].copy()
    lab[0, 5] = 256          # == vocab
    lab[0, 9] = 1 << 30
    lab[0, 12] = -7
    ref_lab = lab.copy()
    ref_lab[(ref_lab < 0) | (ref_lab >= 256)] = -1
    f = inp.f64
    scale = O.target_scale(ref_lab)
    rl, dh, dw = run_head(inp, 32, scale, labels_override=lab)
    _, dh_ref, dw_ref = O.sft_streamed(f["h"], f["w"], ref_lab, 32, scale)
    assert rl[0, 5] == 0.0 and rl[0, 9] == 0.0 and rl[0, 12] == 0.0
    assert np.abs(dh[0, [5, 9, 12]]).max() == 0.0
    assert rel(dh, dh_ref) <= 2e-2 and rel(dw, dw_ref) <= 2e-2


def test_llama3_head_one_partition():
    """The LLaMA3-8B head (d_model 4096, vocab 128256) on one ps_head = 100
    partition: every row loss, every dH row, and sampled dW rows."""
    base = W.HEAD_WORKLOADS["8b_head_sft"]
    wl = W.HeadWorkload(base.name, 1, 100, base.d_model, base.vocab, 100, 10, "bf16", base.seed)
    print(f"[case] {wl.name} one partition", flush=True)
    inp = W.make_head_inputs(wl)
    f = inp.f64
    scale = O.target_scale(f["labels"])
    rl, dh, dw = run_head(inp, 100, scale)
    _, dh_ref, dw_ref = O.sft_streamed(f["h"], f["w"], f["labels"], 100, scale)
    rl_ref = O.row_losses(f["h"], f["w"], f["labels"])
    rows = np.random.default_rng(0).integers(0, base.vocab, 64)
    errs = {"row_loss": rel(rl, rl_ref), "dh": rel(dh, dh_ref),
            "dw_rows": float(np.abs(dw[rows] - dw_ref[rows]).max() / np.abs(dw_ref).max())}
    print(errs, flush=True)
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)


def test_full_size_sampled():
    """The benchmark's workload at full size (T = 16384, ps_head = 100), run as
    the benchmark runs it, partition by partition: sampled row losses and dH
    rows against the oracle computed row by row, and the last (ragged, 84-row)
    partition's weight-gradient increment (dW after it minus dW before it)
    against the oracle's dW of that partition, on sampled vocabulary rows
    including every label of the partition."""
    import torch
    from sequence_chunked_exact_amd import binding as Bn
    wl = W.HEAD_WORKLOADS["8b_head_sft"]
    print(f"[case] {wl.name} full size", flush=True)
    inp = W.make_head_inputs(wl, keep_f64=False)
    lab = inp.raw["labels"]
    scale = 1.0 / float((lab >= 0).sum())
    dev = "cuda:0"
    h_d = W.to_torch(inp.raw["h"], dev)
    w_d = W.to_torch(inp.raw["w"], dev)
    labels = torch.from_numpy(np.ascontiguousarray(lab)).to(dev)
    B, T, dm = h_d.shape
    V = w_d.shape[0]
    wt = torch.empty(dm, V, dtype=h_d.dtype, device=dev)
    row_loss = torch.full((B, T), float("nan"), device=dev)
    dh_d = torch.full((B, T, dm), float("nan"), device=dev)
    dw_d = torch.zeros(V, dm, device=dev)
    ws = Bn.lm_head_sft_workspace(h_d, w_d, wl.ps)
    Bn.lm_head_transpose(w_d, wt)
    starts = list(range(0, T, wl.ps))
    last = starts[-1]
    for s0 in starts:
        if s0 == last:
            torch.cuda.synchronize()
            before = dw_d.cpu()
        Bn.lm_head_sft_partition(h_d, w_d, wt, labels, row_loss, dh_d, dw_d, row_start=s0, rows=min(wl.ps, T - s0),
                                 loss_scale=scale, workspace=ws)
    torch.cuda.synchronize()
    inc = (dw_d.cpu() - before).double().numpy()
    rl = row_loss.cpu().double().numpy()
    dh = dh_d.cpu().double().numpy()
    assert np.isfinite(rl).all() and np.isfinite(dh).all()
    h = W.bf16_bits_to_f64(inp.raw["h"])
    w = W.bf16_bits_to_f64(inp.raw["w"])
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, wl.prompt - 1, wl.prompt, T - 1], rng.integers(0, T, 8)]))
    for t in rows:
        _, dh_t, _ = O.sft_partition(h, w, lab, slice(t, t + 1), scale, with_dw=False)
        rl_t = O.row_losses(h[:, t:t + 1], w, lab[:, t:t + 1])
        e_l = abs(rl[0, t] - rl_t[0, 0]) / max(abs(rl_t[0, 0]), 1e-30)
        e_h = rel(dh[0, t], dh_t[0, 0]) if lab[0, t] >= 0 else float(np.abs(dh[0, t]).max())
        print("row", t, f"{e_l:.2e} {e_h:.2e}", flush=True)
        assert e_l <= 2e-2 and e_h <= 2e-2
    _, _, dw_last = O.sft_partition(h, w, lab, slice(last, T), scale)
    vs = np.union1d(lab[0, last:][lab[0, last:] >= 0], rng.integers(0, V, 64))
    e = float(np.abs(inc[vs] - dw_last[vs]).max() / np.abs(dw_last).max())
    print("last partition dW increment", f"{e:.2e}", flush=True)
    assert e <= 2e-2


def _device_head(inp, dev="cuda:0"):
    import torch
    from sequence_chunked_exact_amd import binding as Bn
    h = W.to_torch(inp.raw["h"], dev)
    w = W.to_torch(inp.raw["w"], dev)
    labels = torch.from_numpy(np.ascontiguousarray(inp.raw["labels"])).to(dev)
    B, T, dm = h.shape
    V = w.shape[0]
    wt = torch.empty(dm, V, dtype=h.dtype, device=dev)
    Bn.lm_head_transpose(w, wt)
    return Bn, torch, h, w, wt, labels, torch.zeros(B, T, device=dev), torch.zeros(B, T, dm, device=dev), \
        torch.zeros(V, dm, device=dev)


def test_grpo_weighted_rows():
    """GRPO's on-policy objective through per-position weights A_i / (G |o_i|)."""
    wl = W.HeadWorkload("grpo", 3, 96, 128, 512, 40, 12, "bf16", seed=37)
    inp = W.make_head_inputs(wl)
    lab = inp.raw["labels"]
    lab[2, 80:] = -1                                   # a shorter response
    adv = np.array([0.8, -1.1, 0.3])
    n = (lab >= 0).sum(axis=1)
    weight = np.where(lab >= 0, (adv / (3 * n))[:, None], 0.0).astype(np.float32)
    Bn, torch, h, w, wt, labels, row_loss, dh, dw = _device_head(inp)
    labels.copy_(torch.from_numpy(lab))
    wd = torch.from_numpy(weight).to(h.device)
    Bn.lm_head_sft(h, w, wt, labels, row_loss, dh, dw, loss_scale=1.0, ps=wl.ps, dw_group=2, row_weight=wd)
    torch.cuda.synchronize()
    f = inp.f64
    loss_ref, dh_ref, dw_ref = O.grpo_dense(f["h"], f["w"], lab, adv)
    loss = float((weight.astype(np.float64) * row_loss.cpu().double().numpy()).sum())
    errs = {"loss": abs(loss - loss_ref) / abs(loss_ref), "dh": rel(dh.cpu().double().numpy(), dh_ref),
            "dw": rel(dw.cpu().double().numpy(), dw_ref)}
    print("grpo", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] <= 1e-3 and errs["dh"] <= 2e-2 and errs["dw"] <= 2e-2


@pytest.mark.parametrize("offset", [0.0, 3.0])
def test_dpo_scalar_correction(offset):
    """DPO on one preference pair: a sweep with weights +1 / -1, then the final
    scalar c = beta sigmoid(-beta margin) from the accumulated log-probabilities."""
    wl = W.HeadWorkload("dpo", 2, 80, 128, 448, 32, 16, "bf16", seed=41)
    inp = W.make_head_inputs(wl)
    lab = inp.raw["labels"]
    f = inp.f64
    lp = -O.row_losses(f["h"], f["w"], lab).sum(axis=1)
    ref = np.array([lp[0] - offset, lp[1] + offset])      # margin 2 * offset
    beta = 0.2
    Bn, torch, h, w, wt, labels, row_loss, dh, dw = _device_head(inp)
    weight = torch.tensor([[1.0], [-1.0]], device=h.device).expand(2, lab.shape[1]).contiguous()
    Bn.lm_head_sft(h, w, wt, labels, row_loss, dh, dw, loss_scale=1.0, ps=wl.ps, dw_group=2, row_weight=weight)
    loss, c = Bn.lm_head_dpo_finish(row_loss, dh, dw, w, ref_logp=ref, beta=beta)
    torch.cuda.synchronize()
    loss_ref, dh_ref, dw_ref, c_ref = O.dpo_dense(f["h"], f["w"], lab, ref, beta)
    errs = {"loss": abs(loss - loss_ref) / abs(loss_ref), "c": abs(c - c_ref) / c_ref,
            "dh": rel(dh.cpu().double().numpy(), dh_ref), "dw": rel(dw.cpu().double().numpy(), dw_ref)}
    print("dpo", offset, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert errs["loss"] <= 2e-3 and errs["c"] <= 2e-3 and errs["dh"] <= 2e-2 and errs["dw"] <= 2e-2


def test_dpo_two_pairs_accumulated_by_the_documented_pattern():
    """lm_head_dpo_finish scales all of dw, so the header asks each pair to be swept
    into a zeroed buffer, finished, then added to the accumulator. Two pairs done
    that way give the sum of the two pairs' DPO weight gradients."""
    Bn = None
    total_ref = None
    acc = None
    beta = 0.3
    for offset in (1.0, -2.0):   # two pairs on one head: different margins, so different c
        wl = W.HeadWorkload("dpo", 2, 80, 128, 448, 32, 16, "bf16", seed=41)
        inp = W.make_head_inputs(wl)
        lab = inp.raw["labels"]
        f = inp.f64
        lp = -O.row_losses(f["h"], f["w"], lab).sum(axis=1)
        ref = np.array([lp[0] - offset, lp[1] + offset])
        Bn, torch, h, w, wt, labels, row_loss, dh, dw = _device_head(inp)
        dw.zero_()
        weight = torch.tensor([[1.0], [-1.0]], device=h.device).expand(2, lab.shape[1]).contiguous()
        Bn.lm_head_sft(h, w, wt, labels, row_loss, dh, dw, loss_scale=1.0, ps=wl.ps, dw_group=2, row_weight=weight)
        Bn.lm_head_dpo_finish(row_loss, dh, dw, w, ref_logp=ref, beta=beta)
        acc = dw.clone() if acc is None else acc + dw
        _, _, dw_ref, _ = O.dpo_dense(f["h"], f["w"], lab, ref, beta)
        total_ref = dw_ref if total_ref is None else total_ref + dw_ref
    torch.cuda.synchronize()
    e = rel(acc.cpu().double().numpy(), total_ref)
    print("dpo two pairs dw", f"{e:.2e}", flush=True)
    assert e <= 2e-2
