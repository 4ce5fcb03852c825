"""Pins for the float64 stack oracle (oracle.stack), each independent of the
oracle's own code path:

- the dense gradient of the attention stack against float64 torch.autograd
  of the same model written directly, and against central finite differences;
- SeCO's exactness: the chunked sweep over every chunk with gamma = 1 equals
  the dense gradient (a different evaluation order reaching the same sum);
- for one layer, the expectation over all t-subsets equals the closed form
  built from per-chunk and per-pair terms with the survival probabilities of
  sampling without replacement, t/k for one chunk and t(t-1)/(k(k-1)) for a
  pair (SeCO/SpaCO review, major comment on Section 5: a chain through n
  distinct chunks survives with probability (t)_n/(k)_n);
- a relayed chain hops to a strictly lower layer each time, so for a fixed
  subset the estimate is a polynomial in gamma of degree at most L.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import projection as P
from oracle import stack as S


def model(L=2, B=1, T=12, Hq=2, Hkv=1, d=4, seed=0):
    rng = np.random.default_rng(seed)
    dm = Hq * d
    h0 = rng.standard_normal((B, T, dm))
    weights = [(rng.standard_normal((dm, Hq * d)) * 0.4, rng.standard_normal((dm, Hkv * d)) * 0.4,
                rng.standard_normal((dm, Hkv * d)) * 0.4) for _ in range(L)]
    y = rng.standard_normal((B, T, dm))
    return h0, weights, y, Hq, Hkv, 1.0 / np.sqrt(d)


def loss(h0, weights, y, Hq, Hkv, scale):
    _, hL = S.stack_forward(h0, weights, Hq, Hkv, scale)
    return float((hL * y).sum())


def test_dense_matches_torch_autograd():
    h0, weights, y, Hq, Hkv, sc = model(L=3, B=2, seed=1)
    B, T, dm = h0.shape
    d = dm // Hq
    th = torch.tensor(h0, requires_grad=True)
    tw = [[torch.tensor(w, requires_grad=True) for w in wl] for wl in weights]
    h = th
    mask = torch.ones(T, T, dtype=torch.bool).triu(1)
    for wq, wk, wv in tw:
        q = (h @ wq).reshape(B, T, Hq, d).permute(0, 2, 1, 3)
        k = (h @ wk).reshape(B, T, Hkv, d).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
        v = (h @ wv).reshape(B, T, Hkv, d).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
        p = torch.softmax((sc * q @ k.transpose(-1, -2)).masked_fill(mask, float("-inf")), dim=-1)
        h = h + (p @ v).permute(0, 2, 1, 3).reshape(B, T, dm)
    (h * torch.tensor(y)).sum().backward()
    grads, dh0 = S.stack_dense_grad(h0, weights, y, Hq, Hkv, sc)
    np.testing.assert_allclose(dh0, th.grad.numpy(), rtol=1e-10, atol=1e-11)
    for l in range(len(weights)):
        for i in range(3):
            np.testing.assert_allclose(grads[l][i], tw[l][i].grad.numpy(), rtol=1e-10, atol=1e-11)


def test_dense_matches_finite_differences():
    h0, weights, y, Hq, Hkv, sc = model(L=2, seed=2)
    grads, dh0 = S.stack_dense_grad(h0, weights, y, Hq, Hkv, sc)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for l, i in ((0, 1), (0, 2), (1, 0), (0, 0)):
        w = weights[l][i]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in w.shape)
            wp, wm = [list(x) for x in weights], [list(x) for x in weights]
            wp[l][i] = w.copy()
            wp[l][i][idx] += eps
            wm[l][i] = w.copy()
            wm[l][i][idx] -= eps
            fd = (loss(h0, wp, y, Hq, Hkv, sc) - loss(h0, wm, y, Hq, Hkv, sc)) / (2 * eps)
            assert abs(fd - grads[l][i][idx]) <= 1e-6 * max(1.0, abs(fd)), (l, i, idx)
    for _ in range(4):
        idx = tuple(int(rng.integers(0, s)) for s in h0.shape)
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += eps
        hm[idx] -= eps
        fd = (loss(hp, weights, y, Hq, Hkv, sc) - loss(hm, weights, y, Hq, Hkv, sc)) / (2 * eps)
        assert abs(fd - dh0[idx]) <= 1e-6 * max(1.0, abs(fd))


@pytest.mark.parametrize("L,T,C", [(1, 12, 3), (2, 12, 3), (3, 10, 4)])
def test_seco_sweep_is_exact(L, T, C):
    h0, weights, y, Hq, Hkv, sc = model(L=L, T=T, seed=3)
    k = -(-T // C)
    grads, dh0 = S.stack_dense_grad(h0, weights, y, Hq, Hkv, sc)
    est, edh0 = S.spaco_estimate(h0, weights, y, Hq, Hkv, sc, C, range(k), 1.0)
    np.testing.assert_allclose(edh0, dh0, rtol=1e-11, atol=1e-12)
    for l in range(L):
        for i in range(3):
            np.testing.assert_allclose(est[l][i], grads[l][i], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("t,gamma", [(2, 2.0), (3, 4.0 / 3.0), (1, 4.0)])
def test_one_layer_expectation_closed_form(t, gamma):
    h0, weights, y, Hq, Hkv, sc = model(L=1, T=12, seed=4)
    C, k = 3, 4
    (wq, wk, wv), = weights
    q, kk, v = P.qkv_forward(h0, wq, wk, wv, Hq, Hkv)
    direct = None
    pairs = None

    def proj(gq, gk, gv):
        dwq, dwk, dwv, dh = P.qkv_backward(h0, wq, wk, wv, gq, gk, gv)
        return [dwq, dwk, dwv, dh]

    def add(acc, x):
        return x if acc is None else [a + b for a, b in zip(acc, x)]

    for j in range(k):
        rows = np.arange(j * C, (j + 1) * C)
        do = np.zeros(q.shape)
        do[:, :, rows] = P.cols_to_heads(y, Hq)[:, :, rows]
        dq, dk, dv = A.backward(q, kk, v, do, sc, rows=rows)
        own = np.zeros(12, bool)
        own[rows] = True
        z = np.zeros_like
        direct = add(direct, proj(np.where(own[None, None, :, None], dq, 0), np.where(own[None, None, :, None], dk, 0),
                                  np.where(own[None, None, :, None], dv, 0)))
        for i in range(j):
            ri = np.zeros(12, bool)
            ri[i * C:(i + 1) * C] = True
            m = ri[None, None, :, None]
            pairs = add(pairs, proj(z(dq), np.where(m, dk, 0), np.where(m, dv, 0)))
    p1 = t / k
    p2 = t * (t - 1) / (k * (k - 1))
    closed = [p1 * a + p2 * gamma * b for a, b in zip(direct, pairs)]
    closed[3] = closed[3] + p1 * y  # the residual path: dJ_j/dH_0 = Y on chunk j's rows
    (ew,), edh = S.spaco_expectation(h0, weights, y, Hq, Hkv, sc, C, t, gamma)
    for i in range(3):
        np.testing.assert_allclose(ew[i], closed[i], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(edh, closed[3], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2])
def test_estimate_is_polynomial_in_gamma_of_degree_at_most_L(L):
    h0, weights, y, Hq, Hkv, sc = model(L=L, T=12, seed=5)
    sub = (0, 2, 3)
    vals = [S.spaco_estimate(h0, weights, y, Hq, Hkv, sc, 3, sub, g) for g in (0.5, 1.0, 1.5, 2.0)]
    flat = [np.concatenate([np.ravel(x) for gl in v[0] for x in gl] + [np.ravel(v[1])]) for v in vals]
    # the (L+1)-th finite difference over equally spaced gamma vanishes
    diff = flat
    for _ in range(L + 1):
        diff = [b - a for a, b in zip(diff, diff[1:])]
    scale = max(np.abs(f).max() for f in flat)
    assert np.abs(diff[0]).max() <= 1e-10 * scale
    if L == 2:  # and degree L is reached: two-hop chains exist
        d2 = [b - a for a, b in zip(flat, flat[1:])]
        d2 = [b - a for a, b in zip(d2, d2[1:])]
        assert np.abs(d2[0]).max() > 1e-6 * scale


def test_unselected_chunks_get_no_input_gradient():
    h0, weights, y, Hq, Hkv, sc = model(L=2, T=12, seed=6)
    _, dh0 = S.spaco_estimate(h0, weights, y, Hq, Hkv, sc, 3, (1, 3), 4.0)
    assert not dh0[:, 0:3].any() and not dh0[:, 6:9].any()
    assert dh0[:, 3:6].any() and dh0[:, 9:12].any()


def test_expectation_enumerates_every_subset_once():
    # With t = k the only subset is everything: expectation = SeCO = dense.
    h0, weights, y, Hq, Hkv, sc = model(L=2, T=9, seed=7)
    grads, dh0 = S.stack_dense_grad(h0, weights, y, Hq, Hkv, sc)
    ew, edh = S.spaco_expectation(h0, weights, y, Hq, Hkv, sc, 3, 3, 1.0)
    np.testing.assert_allclose(edh, dh0, rtol=1e-11, atol=1e-12)
    assert len(list(itertools.combinations(range(3), 3))) == 1
