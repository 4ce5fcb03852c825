"""Pins for the float64 LM-head SFT oracle (oracle.lm_head), each independent
of its code path: torch's float64 cross_entropy with autograd, central finite
differences, the closed form at zero weights (uniform softmax: loss ln V, dh =
0, dW = scale * sum (1/V - onehot) h^T), explicit loops on a tiny case, and
partition invariance of the streamed form (StreamBP review, Eq. (1)).
"""
import numpy as np
import pytest
import torch

from oracle import lm_head as H


def case(B=2, T=9, dm=5, V=7, seed=0, ignore=(1, 4)):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, T, dm))
    w = rng.standard_normal((V, dm)) * 0.7
    y = rng.integers(0, V, (B, T))
    for t in ignore:
        y[0, t] = -1
    return h, w, y


def test_matches_torch_cross_entropy():
    h, w, y = case()
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    z = th @ tw.T
    loss = torch.nn.functional.cross_entropy(z.reshape(-1, w.shape[0]), torch.tensor(y).reshape(-1),
                                             ignore_index=-1, reduction="mean")
    loss.backward()
    l, dh, dw = H.sft_dense(h, w, y)
    assert abs(l - loss.item()) <= 1e-12 * abs(loss.item())
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_finite_differences():
    h, w, y = case(seed=1)
    _, dh, dw = H.sft_dense(h, w, y)
    rng = np.random.default_rng(2)
    eps = 1e-6
    for x, g, name in ((h, dh, "h"), (w, dw, "w")):
        for _ in range(5):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = (xp, w) if name == "h" else (h, xp)
            args_m = (xm, w) if name == "h" else (h, xm)
            fd = (H.sft_dense(*args_p, y)[0] - H.sft_dense(*args_m, y)[0]) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx)


def test_zero_weights_closed_form():
    h, w, y = case(seed=3)
    V = w.shape[0]
    w0 = np.zeros_like(w)
    l, dh, dw = H.sft_dense(h, w0, y)
    assert abs(l - np.log(V)) < 1e-12
    assert np.abs(dh).max() == 0.0
    scale = 1.0 / (y >= 0).sum()
    ref = np.zeros_like(w)
    for b in range(h.shape[0]):
        for t in range(h.shape[1]):
            if y[b, t] < 0:
                continue
            g = np.full(V, 1.0 / V)
            g[y[b, t]] -= 1.0
            ref += scale * np.outer(g, h[b, t])
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-14)


def test_loss_by_explicit_loops():
    h, w, y = case(B=1, T=4, dm=3, V=4, seed=4, ignore=(2,))
    l, _, _ = H.sft_dense(h, w, y)
    total, n = 0.0, 0
    for t in range(4):
        if y[0, t] < 0:
            continue
        z = [sum(w[v, c] * h[0, t, c] for c in range(3)) for v in range(4)]
        total += np.log(sum(np.exp(zz) for zz in z)) - z[y[0, t]]
        n += 1
    assert abs(l - total / n) < 1e-12
    rl = H.row_losses(h, w, y)
    assert rl[0, 2] == 0.0 and abs(rl.sum() - total) < 1e-12


@pytest.mark.parametrize("ps", [1, 3, 4, 100])
def test_streaming_is_partition_invariant(ps):
    h, w, y = case(T=11, seed=5)
    l, dh, dw = H.sft_dense(h, w, y)
    ls, dhs, dws = H.sft_streamed(h, w, y, ps)
    assert abs(ls - l) <= 1e-12 * abs(l)
    np.testing.assert_allclose(dhs, dh, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dws, dw, rtol=1e-12, atol=1e-15)


def test_no_targets_gives_zero():
    h, w, y = case(seed=6)
    y[:] = -1
    l, dh, dw = H.sft_dense(h, w, y)
    assert l == 0.0 and not dh.any() and not dw.any()


def test_grpo_matches_torch_autograd():
    h, w, y = case(B=3, T=8, seed=8, ignore=(0, 1))
    y[2, :3] = -1
    adv = np.array([0.7, -1.2, 0.4])
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    logp = torch.log_softmax(th @ tw.T, dim=-1)
    ty = torch.tensor(y)
    tgt = ty >= 0
    lp = torch.gather(logp, -1, ty.clamp(min=0)[..., None])[..., 0] * tgt
    loss = -(torch.tensor(adv)[:, None] * lp / tgt.sum(dim=1, keepdim=True)).sum() / 3
    loss.backward()
    l, dh, dw = H.grpo_dense(h, w, y, adv)
    assert abs(l - loss.item()) <= 1e-12 * abs(loss.item())
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_grpo_with_equal_advantages_and_lengths_is_scaled_sft():
    h, w, y = case(B=2, T=6, seed=9, ignore=())
    l, dh, dw = H.grpo_dense(h, w, y, np.array([1.0, 1.0]))
    ls, dhs, dws = H.sft_dense(h, w, y)
    assert abs(l - ls) < 1e-12
    np.testing.assert_allclose(dh, dhs, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dw, dws, rtol=1e-12, atol=1e-15)


def test_dpo_matches_torch_autograd_and_finite_differences():
    h, w, y = case(B=2, T=7, seed=10, ignore=(0,))
    y[1, :2] = -1
    ref = np.array([-20.0, -21.5])
    beta = 0.3
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    logp = torch.log_softmax(th @ tw.T, dim=-1)
    ty = torch.tensor(y)
    lp = (torch.gather(logp, -1, ty.clamp(min=0)[..., None])[..., 0] * (ty >= 0)).sum(dim=1)
    margin = (lp[0] - ref[0]) - (lp[1] - ref[1])
    loss = -torch.nn.functional.logsigmoid(beta * margin)
    loss.backward()
    l, dh, dw, c = H.dpo_dense(h, w, y, ref, beta)
    assert abs(l - loss.item()) <= 1e-12 * abs(loss.item())
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-13)
    eps = 1e-6
    idx = (1, 3)
    wp, wm = w.copy(), w.copy()
    wp[idx] += eps
    wm[idx] -= eps
    fd = (H.dpo_dense(h, wp, y, ref, beta)[0] - H.dpo_dense(h, wm, y, ref, beta)[0]) / (2 * eps)
    assert abs(fd - dw[idx]) <= 1e-7 * max(1.0, abs(fd))


def test_dpo_at_zero_margin():
    # margin 0: loss ln 2 and c = beta / 2
    h, w, y = case(B=2, T=5, seed=11, ignore=())
    logp = -H.row_losses(h, w, y)
    ref = logp.sum(axis=1)
    l, _, _, c = H.dpo_dense(h, w, y, ref, 0.5)
    assert abs(l - np.log(2.0)) < 1e-12 and abs(c - 0.25) < 1e-15
