"""Pins for the float64 oracle, each independent of the oracle's own code.

Every check here fixes the oracle to something other than itself: central
finite differences, float64 torch.autograd on the naive masked-softmax formula,
closed forms, invariants, and an independent online-softmax chunked evaluation
(the chunk-sum identity of StreamBP's Eq. (1), StreamBP review "What carries
the argument"; float64 agreement to 12+ decimals is the SeCO standard,
SeCO/SpaCO review, Referee Report summary, Appendix D).
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small(T=9, Hq=4, Hkv=2, d=5, B=1, seed=0):
    q = rand((B, Hq, T, d), seed)
    k = rand((B, Hkv, T, d), seed + 1)
    v = rand((B, Hkv, T, d), seed + 2)
    do = rand((B, Hq, T, d), seed + 3)
    return q, k, v, do


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("Hq,Hkv,scale,block", [(2, 1, 0.7, 4), (2, 2, 1.0, 3), (3, 1, 0.5, 100),
                                                (2, 1, -0.6, 4)])
def test_finite_differences(Hq, Hkv, scale, block):
    q, k, v, do = small(T=6, Hq=Hq, Hkv=Hkv, d=3, seed=11)

    def loss(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, scale, block=block)
        return float((do * o).sum())

    dq, dk, dv = A.backward(q, k, v, do, scale, block=block)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp; lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm; lm = loss(args["q"], args["k"], args["v"])
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / np.abs(fd).max()
        assert err < 1e-6, (name, err)


# ---------------------------------------------------------------- library cross-check
def torch_reference(q, k, v, do, scale):
    """Naive masked softmax in float64 autograd; GQA by repeating kv heads."""
    G = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    T = q.shape[2]
    s = scale * tq @ kk.transpose(-1, -2)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.softmax(s, dim=-1) @ vv
    o.backward(torch.tensor(do))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


@pytest.mark.parametrize("T,Hq,Hkv,d,B,scale,block", [
    (9, 4, 2, 5, 1, 0.8, 4),
    (33, 8, 2, 16, 2, 0.25, 8),
    (70, 3, 3, 7, 1, 1.0, 256),
    (1, 2, 1, 4, 1, 1.0, 4),
    (40, 4, 1, 8, 1, -0.9, 16),       # negative scale: the softmax favours anti-aligned keys
])
def test_torch_autograd_crosscheck(T, Hq, Hkv, d, B, scale, block):
    q, k, v, do = small(T=T, Hq=Hq, Hkv=Hkv, d=d, B=B, seed=T)
    o, lse = A.forward(q, k, v, scale, block=block)
    dq, dk, dv = A.backward(q, k, v, do, scale, block=block)
    ro, rlse, rdq, rdk, rdv = torch_reference(q, k, v, do, scale)
    for a, b in ((o, ro), (lse, rlse), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


# ---------------------------------------------------------------- closed forms
def test_zero_keys_closed_form():
    T, Hq, Hkv, d = 12, 4, 2, 6
    q, _, v, do = small(T=T, Hq=Hq, Hkv=Hkv, d=d, seed=5)
    k = np.zeros_like(v)
    o, lse = A.forward(q, k, v, 0.9, block=5)
    dq, dk, dv = A.backward(q, k, v, do, 0.9, block=5)
    r = np.arange(T)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        running_mean = np.cumsum(v[0, g], axis=0) / (r + 1)[:, None]
        assert np.allclose(o[0, h], running_mean, atol=1e-14, rtol=0)
        assert np.allclose(lse[0, h], np.log(r + 1), atol=1e-14, rtol=0)
    assert np.abs(dq).max() == 0.0
    for g in range(Hkv):
        want = np.zeros((T, d))
        for h in range(g * G, (g + 1) * G):
            w = do[0, h] / (r + 1)[:, None]
            want += np.cumsum(w[::-1], axis=0)[::-1]       # sum over r >= j
        assert np.allclose(dv[0, g], want, atol=1e-13, rtol=0)


def test_single_token_closed_form():
    q, k, v, do = small(T=1, Hq=2, Hkv=1, d=4, seed=9)
    o, lse = A.forward(q, k, v, 1.3)
    dq, dk, dv = A.backward(q, k, v, do, 1.3)
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[0, 1], v[0, 0])
    assert np.allclose(lse[0, :, 0], 1.3 * (q[0, :, 0] @ k[0, 0, 0]), atol=1e-15)
    assert np.allclose(dv[0, 0, 0], do[0, 0, 0] + do[0, 1, 0], atol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


# ---------------------------------------------------------------- invariants
def test_rows_normalise():
    q, k, v, do = small(T=20, seed=2)
    _, lse = A.forward(q, k, v, 0.6, block=7)
    G = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        s = 0.6 * q[0, h] @ k[0, h // G].T
        for r in range(20):
            tot = np.exp(s[r, :r + 1] - lse[0, h, r]).sum()
            assert abs(tot - 1.0) < 1e-12


def test_shift_and_scale_invariance():
    q, k, v, do = small(T=17, seed=3)
    c = rand((5,), 77)
    o, lse = A.forward(q, k, v, 0.7)
    grads = A.backward(q, k, v, do, 0.7)
    o2, lse2 = A.forward(q, k + c, v, 0.7)
    G = q.shape[1] // k.shape[1]
    assert np.allclose(o, o2, atol=1e-13, rtol=0)
    assert np.allclose(lse2 - lse, 0.7 * (q @ c), atol=1e-12, rtol=0)
    dq2, _, dv2 = A.backward(q, k + c, v, do, 0.7)
    assert np.allclose(dq2, grads[0], atol=1e-12) and np.allclose(dv2, grads[2], atol=1e-12)
    a = 2.5
    o3, lse3 = A.forward(a * q, k, v, 0.7 / a)
    assert np.allclose(o3, o, atol=1e-13) and np.allclose(lse3, lse, atol=1e-12)
    del G


def test_gradient_column_sums():
    # sum_j dS_rj = 0 for every row, so dK summed over keys vanishes; rows of P
    # sum to one, so dV summed over keys equals dO summed over the group's rows.
    q, k, v, do = small(T=23, Hq=4, Hkv=2, seed=4)
    dq, dk, dv = A.backward(q, k, v, do, 0.9, block=6)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    want = do.reshape(1, 2, 2, 23, 5).sum(axis=(2, 3))
    assert np.allclose(dv.sum(axis=2), want, atol=1e-12)


def test_gqa_matches_repeated_heads():
    q, k, v, do = small(T=15, Hq=6, Hkv=2, seed=6)
    G = 3
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse = A.forward(q, k, v, 0.8)
    dq, dk, dv = A.backward(q, k, v, do, 0.8)
    o_m, lse_m = A.forward(q, kr, vr, 0.8)
    dq_m, dk_m, dv_m = A.backward(q, kr, vr, do, 0.8)
    assert np.allclose(o, o_m, atol=1e-15) and np.allclose(lse, lse_m, atol=1e-15)
    assert np.allclose(dq, dq_m, atol=1e-14)
    assert np.allclose(dk, dk_m.reshape(1, 2, 3, 15, 5).sum(axis=2), atol=1e-13)
    assert np.allclose(dv, dv_m.reshape(1, 2, 3, 15, 5).sum(axis=2), atol=1e-13)


# ---------------------------------------------------------------- chunk identity
def online_chunk(qc, kp, vp, doc, scale, start, tile):
    """One chunk by a different algorithm: streaming key tiles with a running
    max, and the dO.O row identity for the softmax-Jacobian term."""
    C, d = qc.shape
    pos = start + np.arange(C)
    m = np.full(C, -np.inf); l = np.zeros(C); acc = np.zeros((C, d))
    for j0 in range(0, kp.shape[0], tile):
        kt, vt = kp[j0:j0 + tile], vp[j0:j0 + tile]
        s = scale * qc @ kt.T
        s[(j0 + np.arange(kt.shape[0]))[None, :] > pos[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)
        e = np.exp(s - m_new[:, None])
        l = l * alpha + e.sum(axis=1)
        acc = acc * alpha[:, None] + e @ vt
        m = m_new
    o = acc / l[:, None]
    lse = m + np.log(l)
    delta = (doc * o).sum(axis=1)
    dq = np.zeros_like(qc); dk = np.zeros_like(kp); dv = np.zeros_like(vp)
    for j0 in range(0, kp.shape[0], tile):
        kt, vt = kp[j0:j0 + tile], vp[j0:j0 + tile]
        s = scale * qc @ kt.T
        p = np.exp(s - lse[:, None])
        p[(j0 + np.arange(kt.shape[0]))[None, :] > pos[:, None]] = 0.0
        ds = p * (doc @ vt.T - delta[:, None])
        dq += scale * ds @ kt
        dk[j0:j0 + tile] = scale * ds.T @ qc
        dv[j0:j0 + tile] = p.T @ doc
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("T,C,Hq,Hkv", [(40, 12, 2, 1), (64, 16, 4, 4), (37, 37, 2, 2)])
def test_chunk_sum_identity(T, C, Hq, Hkv):
    q, k, v, do = small(T=T, Hq=Hq, Hkv=Hkv, d=8, seed=T + C)
    scale = 1 / math.sqrt(8)
    o, lse = A.forward(q, k, v, scale, block=5)
    dq, dk, dv = A.backward(q, k, v, do, scale, block=5)
    G = Hq // Hkv
    co, clse, cdq = np.zeros_like(o), np.zeros_like(lse), np.zeros_like(dq)
    cdk, cdv = np.zeros_like(dk), np.zeros_like(dv)
    for s0 in reversed(range(0, T, C)):
        c = min(C, T - s0); L = s0 + c
        for h in range(Hq):
            g = h // G
            r = online_chunk(q[0, h, s0:L], k[0, g, :L], v[0, g, :L], do[0, h, s0:L], scale, s0, 7)
            co[0, h, s0:L], clse[0, h, s0:L], cdq[0, h, s0:L] = r[0], r[1], r[2]
            cdk[0, g, :L] += r[3]
            cdv[0, g, :L] += r[4]
    for a, b in ((co, o), (clse, lse), (cdq, dq), (cdk, dk), (cdv, dv)):
        assert np.abs(a - b).max() < 1e-12


def test_row_subsets_add_up():
    q, k, v, do = small(T=30, Hq=4, Hkv=2, seed=8)
    full = A.backward(q, k, v, do, 0.5, block=4)
    parts = [A.backward(q, k, v, do, 0.5, rows=np.arange(a, b), block=4)
             for a, b in ((0, 7), (7, 19), (19, 30))]
    for i in range(3):
        assert np.allclose(sum(p[i] for p in parts), full[i], atol=1e-14)
    o, lse = A.forward(q, k, v, 0.5)
    o2, lse2 = A.forward(q, k, v, 0.5, rows=[3, 17, 29], heads=[1])
    assert np.array_equal(o2[0, 1, [3, 17, 29]], o[0, 1, [3, 17, 29]])
    assert np.abs(o2[0, 0]).max() == 0.0


# ---------------------------------------------------------------- sparse estimator
def test_sparse_exhaustive_subsets_unbiased():
    # With one layer the keys/values are leaves: each chunk is kept with
    # probability t/k, so the mean over all t-subsets of the k/t-scaled
    # gradient is the dense gradient.
    T, C, k_chunks, t = 32, 8, 4, 2
    q, k, v, do = small(T=T, Hq=4, Hkv=2, d=6, seed=12)
    dense = A.backward(q, k, v, do, 0.7)
    subsets = list(itertools.combinations(range(k_chunks), t))
    acc = [np.zeros_like(x) for x in dense]
    for sub in subsets:
        g = A.sparse_backward(q, k, v, do, 0.7, C, sub, k_chunks)
        for a, x in zip(acc, g):
            a += x
    for a, x in zip(acc, dense):
        assert np.abs(a / len(subsets) - x).max() < 1e-13


def test_sparse_all_chunks_is_dense():
    q, k, v, do = small(T=20, Hq=2, Hkv=1, d=4, seed=13)
    dense = A.backward(q, k, v, do, 1.0)
    sp = A.sparse_backward(q, k, v, do, 1.0, 6, [0, 1, 2, 3], 4)
    for a, b in zip(sp, dense):
        assert np.allclose(a, b, atol=1e-14)
