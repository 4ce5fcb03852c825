"""Pins for the float64 projection oracle (oracle.projection), each independent
of the oracle's own code: central finite differences of the layer loss,
float64 torch.autograd of the naive layer, explicit loops on tiny shapes, an
identity-weight closed form, and the per-chunk forms of the weight gradients
written in the StreamBP review (major comment 1) summed over chunks.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import projection as P


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def layer(T=7, dm=6, Hq=4, Hkv=2, d=3, B=1, seed=0):
    h = rand((B, T, dm), seed)
    wq = rand((dm, Hq * d), seed + 1, 0.5)
    wk = rand((dm, Hkv * d), seed + 2, 0.5)
    wv = rand((dm, Hkv * d), seed + 3, 0.5)
    do = rand((B, Hq, T, d), seed + 4)
    return h, wq, wk, wv, do


def loss(h, wq, wk, wv, do, Hq, Hkv, scale):
    o, _, _ = P.layer_forward(h, wq, wk, wv, Hq, Hkv, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("which", ["wq", "wk", "wv", "h"])
def test_finite_differences(which):
    Hq, Hkv, scale = 4, 2, 0.7
    h, wq, wk, wv, do = layer(Hq=Hq, Hkv=Hkv)
    grads = dict(zip(["wq", "wk", "wv", "h"], P.layer_backward(h, wq, wk, wv, do, Hq, Hkv, scale)))
    args = {"h": h, "wq": wq, "wk": wk, "wv": wv}
    x = args[which]
    eps = 1e-6
    rng = np.random.default_rng(5)
    for _ in range(6):
        idx = tuple(int(rng.integers(0, s)) for s in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        lp = loss(**{**args, which: xp}, do=do, Hq=Hq, Hkv=Hkv, scale=scale)
        lm = loss(**{**args, which: xm}, do=do, Hq=Hq, Hkv=Hkv, scale=scale)
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - grads[which][idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


def test_matches_torch_autograd():
    Hq, Hkv, d, scale = 4, 2, 3, 0.9
    h, wq, wk, wv, do = layer(T=8, dm=5, Hq=Hq, Hkv=Hkv, d=d, B=2, seed=3)
    th, tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (h, wq, wk, wv))
    B, T, _ = h.shape

    def heads(x, n):
        return x.reshape(B, T, n, d).permute(0, 2, 1, 3)

    q, k, v = heads(th @ tq, Hq), heads(th @ tk, Hkv), heads(th @ tv, Hkv)
    k = k.repeat_interleave(Hq // Hkv, dim=1)
    v = v.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * q @ k.transpose(-1, -2)
    mask = torch.ones(T, T, dtype=torch.bool).triu(1)
    o = torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1) @ v
    (o * torch.tensor(do)).sum().backward()
    dwq, dwk, dwv, dh = P.layer_backward(h, wq, wk, wv, do, Hq, Hkv, scale)
    for mine, ref in ((dwq, tq.grad), (dwk, tk.grad), (dwv, tv.grad), (dh, th.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_projection_by_explicit_loops():
    h, wq, wk, wv, _ = layer(T=4, dm=3, Hq=2, Hkv=1, d=2, B=2, seed=7)
    q, k, v = P.qkv_forward(h, wq, wk, wv, 2, 1)
    B, T, dm = h.shape
    for b in range(B):
        for t in range(T):
            for hh in range(2):
                for c in range(2):
                    ref = sum(h[b, t, m] * wq[m, hh * 2 + c] for m in range(dm))
                    assert abs(q[b, hh, t, c] - ref) < 1e-12
            for c in range(2):
                assert abs(k[b, 0, t, c] - sum(h[b, t, m] * wk[m, c] for m in range(dm))) < 1e-12
                assert abs(v[b, 0, t, c] - sum(h[b, t, m] * wv[m, c] for m in range(dm))) < 1e-12
    # weight gradient by loops: dW[m][n] = sum_b sum_t h[b,t,m] * g[b,t,n]
    g = rand((B, 2, T, 2), 9)
    dwq, _, _, _ = P.qkv_backward(h, wq, wk, wv, g, np.zeros((B, 1, T, 2)), np.zeros((B, 1, T, 2)))
    for m in range(dm):
        for hh in range(2):
            for c in range(2):
                ref = sum(h[b, t, m] * g[b, hh, t, c] for b in range(B) for t in range(T))
                assert abs(dwq[m, hh * 2 + c] - ref) < 1e-12


def test_identity_projection_splits_heads():
    Hq, d, T = 3, 4, 5
    h = rand((1, T, Hq * d), 11)
    eye = np.eye(Hq * d)
    q, k, v = P.qkv_forward(h, eye, eye, eye, Hq, Hq)
    for hh in range(Hq):
        np.testing.assert_array_equal(q[0, hh], h[0, :, hh * d:(hh + 1) * d])
    # dH_in with identity weights is the sum of the three gradients, re-joined
    g = [rand((1, Hq, T, d), 12 + i) for i in range(3)]
    _, _, _, dh = P.qkv_backward(h, eye, eye, eye, *g)
    np.testing.assert_allclose(dh[0], sum(P.heads_to_cols(x)[0] for x in g), rtol=0, atol=1e-13)


def test_chunked_weight_gradients_sum_to_dense():
    # The review's per-chunk forms, dW_k^(i) = H_in^(:i)^T dK^(:i) with dK^(:i)
    # chunk i's contribution over its prefix, and the form used by the library
    # (each chunk's own rows of the accumulated dK), both sum to H_in^T dK.
    Hq, Hkv, d, T, C, scale = 4, 2, 3, 10, 4, 0.8
    h, wq, wk, wv, do = layer(T=T, dm=5, Hq=Hq, Hkv=Hkv, d=d, seed=21)
    q, k, v = P.qkv_forward(h, wq, wk, wv, Hq, Hkv)
    dq, dk, dv = A.backward(q, k, v, do, scale)
    dwq, dwk, dwv, dh = P.qkv_backward(h, wq, wk, wv, dq, dk, dv)
    gk, gq = P.heads_to_cols(dk)[0], P.heads_to_cols(dq)[0]
    hh = h[0]
    per_prefix = np.zeros_like(dwk)
    per_rows = np.zeros_like(dwk)
    per_rows_q = np.zeros_like(dwq)
    for s in range(0, T, C):
        e = min(T, s + C)
        _, dk_i, _ = A.backward(q, k, v, do, scale, rows=np.arange(s, e))
        per_prefix += hh[:e].T @ P.heads_to_cols(dk_i)[0][:e]
        per_rows += hh[s:e].T @ gk[s:e]
        per_rows_q += hh[s:e].T @ gq[s:e]
    np.testing.assert_allclose(per_prefix, dwk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(per_rows, dwk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(per_rows_q, dwq, rtol=1e-12, atol=1e-12)
