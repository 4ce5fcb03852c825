"""Oracle: the language-model head's supervised fine-tuning loss and its
gradients, dense and streamed over sequence partitions, in float64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
only the tests and the benchmark's CPU-baseline leg use it. It shares no code
with the HIP library.

What it computes. StreamBP streams the language-modeling head by partitioning
the logits along the sequence, ps_head = 100 positions at a time, the SFT loss
being separable over positions (StreamBP review, "Core claim"; "Assumptions":
Eq. (3), ps_head = 100). The page does not print Eq. (3); the reading here is
the standard next-token objective: with logits z_t = W h_t (W [vocab][d_model])
and target labels y_t (-1: not a target),

    L = scale * sum_{t: y_t >= 0} (logsumexp(z_t) - z_t[y_t]),  scale = 1 / #targets

    dz_t = scale * (softmax(z_t) - onehot(y_t))   (0 where y_t < 0)
    dh_t = W^T dz_t,      dW = sum_t dz_t h_t^T

Streaming over partitions of the positions gives the same sums (Eq. (1) of the
page: a weight gradient is a sum over output chunks); the loss is the sum of the
partitions' terms. Matrix products are numpy's float64 matmul.
"""
from __future__ import annotations

import numpy as np


def _lse(z):
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def target_scale(labels):
    """1 / number of target positions (0 if there are none)."""
    n = int((np.asarray(labels) >= 0).sum())
    return 1.0 / n if n else 0.0


def sft_partition(h, w, labels, rows, scale, with_dw=True):
    """Loss terms and gradients of the positions ``rows`` (a range of the
    sequence) for every batch entry: (loss, dh over those rows [B, len, d_model],
    dW contribution [vocab, d_model], or None without ``with_dw``)."""
    h = np.asarray(h, dtype=np.float64)[:, rows]
    w = np.asarray(w, dtype=np.float64)
    y = np.asarray(labels)[:, rows]
    z = h @ w.T                                     # [B, len, V]
    lse = _lse(z)
    tgt = y >= 0
    yc = np.where(tgt, y, 0)
    z_y = np.take_along_axis(z, yc[..., None], axis=-1)[..., 0]
    loss = scale * float(np.where(tgt, lse - z_y, 0.0).sum())
    p = np.exp(z - lse[..., None])
    onehot = np.zeros_like(p)
    np.put_along_axis(onehot, yc[..., None], 1.0, axis=-1)
    dz = scale * (p - onehot) * tgt[..., None]
    dh = dz @ w
    dw = sum(dz[b].T @ h[b] for b in range(h.shape[0])) if with_dw else None
    return loss, dh, dw


def sft_dense(h, w, labels, scale=None):
    """(loss, dh [B, T, d_model], dW [vocab, d_model]) over the whole sequence."""
    T = np.asarray(h).shape[1]
    scale = target_scale(labels) if scale is None else scale
    return sft_partition(h, w, labels, slice(0, T), scale)


def sft_streamed(h, w, labels, ps, scale=None):
    """The same quantities accumulated partition by partition (ps positions each)."""
    h = np.asarray(h, dtype=np.float64)
    B, T, dm = h.shape
    scale = target_scale(labels) if scale is None else scale
    loss = 0.0
    dh = np.zeros((B, T, dm))
    dw = np.zeros(np.asarray(w).shape)
    for s in range(0, T, ps):
        rows = slice(s, min(T, s + ps))
        l_i, dh_i, dw_i = sft_partition(h, w, labels, rows, scale)
        loss += l_i
        dh[:, rows] = dh_i
        dw += dw_i
    return loss, dh, dw


def row_losses(h, w, labels):
    """Unscaled per-position loss terms [B, T] (0 where the label is -1)."""
    h = np.asarray(h, dtype=np.float64)
    z = h @ np.asarray(w, dtype=np.float64).T
    y = np.asarray(labels)
    tgt = y >= 0
    z_y = np.take_along_axis(z, np.where(tgt, y, 0)[..., None], axis=-1)[..., 0]
    return np.where(tgt, _lse(z) - z_y, 0.0)


def _logp_rows(h, w, labels):
    """log p(y_t) per position [B, T] (0 where the label is not a target) and the
    softmax P [B, T, V]."""
    h = np.asarray(h, dtype=np.float64)
    z = h @ np.asarray(w, dtype=np.float64).T
    y = np.asarray(labels)
    tgt = y >= 0
    lse = _lse(z)
    z_y = np.take_along_axis(z, np.where(tgt, y, 0)[..., None], axis=-1)[..., 0]
    return np.where(tgt, z_y - lse, 0.0), np.exp(z - lse[..., None]), tgt


def weighted_grads(h, w, labels, weight):
    """dh, dW of sum_t weight_t * (-log p(y_t)) over target positions:
    dz_t = weight_t (softmax(z_t) - onehot(y_t))."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    _, p, tgt = _logp_rows(h, w, labels)
    y = np.where(tgt, np.asarray(labels), 0)
    onehot = np.zeros_like(p)
    np.put_along_axis(onehot, y[..., None], 1.0, axis=-1)
    dz = np.asarray(weight, dtype=np.float64)[..., None] * (p - onehot) * tgt[..., None]
    return dz @ w, sum(dz[b].T @ h[b] for b in range(h.shape[0]))


def grpo_dense(h, w, labels, advantages):
    """GRPO's policy-gradient objective on one group of B sampled responses to a
    prompt (StreamBP review, "Assumptions": Eq. (6), separable over positions).
    The page does not print Eq. (6); the reading is the on-policy form (ratio 1,
    no clipping or KL term): L = -(1/B) sum_i (1/|o_i|) sum_{t in o_i} A_i log p(y_t),
    with o_i the target positions of batch entry i. Returns (L, dh, dW)."""
    logp, _, tgt = _logp_rows(h, w, labels)
    n = np.maximum(tgt.sum(axis=1), 1)
    B = logp.shape[0]
    wt = (np.asarray(advantages, dtype=np.float64) / (B * n))[:, None] * np.ones_like(logp)
    loss = float(-(wt * logp).sum())
    dh, dw = weighted_grads(h, w, labels, wt)
    return loss, dh, dw


def dpo_dense(h, w, labels, ref_logp, beta):
    """DPO on one preference pair, batch entry 0 the chosen response and 1 the
    rejected one (StreamBP review, "Assumptions": Eqs. (8)-(10); the loss is not
    separable but its gradient factorizes with a final scalar). Reading:
    L = -log sigmoid(beta * ((lp_c - ref_c) - (lp_r - ref_r))), lp = sum over the
    response's target positions of log p(y_t). dL/dtheta = c * (grad(-lp_c) -
    grad(-lp_r)), c = beta * sigmoid(-beta * margin): the sum of the per-position
    gradients with weights +1 / -1, multiplied by c once every position is done.
    Returns (L, dh, dW, c)."""
    logp, _, _ = _logp_rows(h, w, labels)
    lp = logp.sum(axis=1)
    margin = (lp[0] - ref_logp[0]) - (lp[1] - ref_logp[1])
    loss = float(np.logaddexp(0.0, -beta * margin))          # -log sigmoid(beta * margin)
    c = beta / (1.0 + np.exp(beta * margin))                 # beta * sigmoid(-beta * margin)
    sign = np.array([1.0, -1.0])[:, None] * np.ones_like(logp)
    dh, dw = weighted_grads(h, w, labels, sign)
    return loss, c * dh, c * dw, c
