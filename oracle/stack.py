"""Oracle: SpaCO's relayed cache gradients across a stack of attention layers,
in float64 on the CPU.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
only the tests and the benchmark's CPU-baseline leg use it. It shares no code
with the HIP library.

The model. The pages define SpaCO on a transformer whose KV caches carry
gradients from later chunks back to earlier ones; a chain of such hops crosses
one layer per hop (SeCO/SpaCO review, "Assumptions": KV-cache chunks of one
layer are independent, so errors move from one cache chunk to another only
between adjacent layers). The smallest model with that structure, used here,
is a stack of L causal attention layers with residual connections:

    Q_l, K_l, V_l = H_l W_q^l, H_l W_k^l, H_l W_v^l      (oracle.projection)
    O_l = causal softmax attention(Q_l, K_l, V_l)        (oracle.attention)
    H_{l+1} = H_l + O_l   (heads side by side: Hq * d = d_model)

with the loss J = sum_j J_j, J_j = <H_L, Y> over chunk j's rows, so dJ/dH_L =
Y. There is no output projection, norm or MLP: those act on each position
alone and move no gradient between chunks.

SpaCO's estimator (Algorithm 2 of the SeCO/SpaCO paper, as the review's major
comments describe it): draw t of the k chunks without replacement (line 4);
for each drawn chunk j, from the last to the first, rebuild its graph with the
earlier chunks' caches as leaves and backpropagate J_j together with the
gradient that later drawn chunks accumulated into chunk j's own cache rows,
that relayed gradient multiplied by k/t (line 7: m_j.grad <- (k/t) m'_j.grad).
The direct term is not scaled. The deployed variant caps the factor at 2
(review, major comment on Section 6.4); gamma is a parameter here. The cache
gradients of chunks that are not drawn are dropped. With every chunk drawn and
gamma = 1 this is SeCO, whose gradient is the dense one.
"""
from __future__ import annotations

import itertools

import numpy as np

from . import attention
from . import projection


def stack_forward(h0, weights, n_q_heads, n_kv_heads, scale):
    """Per layer (H_l, Q_l, K_l, V_l) and the final H_L.

    h0: [B, T, d_model]; weights: list of (W_q, W_k, W_v) per layer."""
    h = np.asarray(h0, dtype=np.float64)
    layers = []
    for wq, wk, wv in weights:
        q, k, v = projection.qkv_forward(h, wq, wk, wv, n_q_heads, n_kv_heads)
        o, _ = attention.forward(q, k, v, scale)
        layers.append((h, q, k, v))
        h = h + projection.heads_to_cols(o)
    return layers, h


def stack_dense_grad(h0, weights, y, n_q_heads, n_kv_heads, scale):
    """dJ/dW per layer [(dW_q, dW_k, dW_v)] and dJ/dH_0 of the whole stack."""
    layers, _ = stack_forward(h0, weights, n_q_heads, n_kv_heads, scale)
    dh = np.asarray(y, dtype=np.float64)
    grads = [None] * len(weights)
    for l in reversed(range(len(weights))):
        h, q, k, v = layers[l]
        wq, wk, wv = weights[l]
        dq, dk, dv = attention.backward(q, k, v, projection.cols_to_heads(dh, n_q_heads), scale)
        dwq, dwk, dwv, dh_proj = projection.qkv_backward(h, wq, wk, wv, dq, dk, dv)
        grads[l] = (dwq, dwk, dwv)
        dh = dh + dh_proj
    return grads, dh


def spaco_estimate(h0, weights, y, n_q_heads, n_kv_heads, scale, chunk, selected, gamma):
    """SpaCO's gradient estimate for the drawn chunks ``selected`` (0-based).

    Returns ([(dW_q, dW_k, dW_v)] per layer, dH_0 with the drawn chunks' rows
    set and the other rows zero)."""
    layers, _ = stack_forward(h0, weights, n_q_heads, n_kv_heads, scale)
    y = np.asarray(y, dtype=np.float64)
    B, T, dm = y.shape
    L = len(weights)
    # accumulated cache gradients m'.grad per layer, all rows
    acc_k = [np.zeros(layers[l][2].shape) for l in range(L)]
    acc_v = [np.zeros(layers[l][3].shape) for l in range(L)]
    grads = [[np.zeros(w.shape) for w in weights[l]] for l in range(L)]
    dh0 = np.zeros((B, T, dm))
    for j in sorted(selected, reverse=True):
        rows = np.arange(j * chunk, min(T, (j + 1) * chunk))
        dh = np.zeros((B, T, dm))
        dh[:, rows] = y[:, rows]                      # dJ_j / dH_L
        for l in reversed(range(L)):
            h, q, k, v = layers[l]
            wq, wk, wv = weights[l]
            # relay: chunk j's own cache rows carry what later drawn chunks
            # accumulated there, multiplied by gamma
            acc_k[l][:, :, rows] *= gamma
            acc_v[l][:, :, rows] *= gamma
            dq, dk, dv = attention.backward(q, k, v, projection.cols_to_heads(dh, n_q_heads), scale, rows=rows)
            acc_k[l] += dk                            # prefix rows [0, end of chunk j)
            acc_v[l] += dv
            # chunk j's projections see dQ of its rows and the (now complete)
            # cache gradient of its rows
            gq = np.zeros_like(dq)
            gk = np.zeros_like(dk)
            gv = np.zeros_like(dv)
            gq[:, :, rows] = dq[:, :, rows]
            gk[:, :, rows] = acc_k[l][:, :, rows]
            gv[:, :, rows] = acc_v[l][:, :, rows]
            dwq, dwk, dwv, dh_proj = projection.qkv_backward(h, wq, wk, wv, gq, gk, gv)
            grads[l][0] += dwq
            grads[l][1] += dwk
            grads[l][2] += dwv
            dh = dh + dh_proj
        dh0[:, rows] = dh[:, rows]
    return [tuple(g) for g in grads], dh0


def spaco_expectation(h0, weights, y, n_q_heads, n_kv_heads, scale, chunk, t, gamma):
    """Expectation of spaco_estimate over all t-subsets of the k chunks (each
    subset equally likely, as in sampling without replacement)."""
    T = np.asarray(y).shape[1]
    k = -(-T // chunk)
    subsets = list(itertools.combinations(range(k), t))
    mean_w, mean_h = None, None
    for sub in subsets:
        g, dh0 = spaco_estimate(h0, weights, y, n_q_heads, n_kv_heads, scale, chunk, sub, gamma)
        if mean_w is None:
            mean_w = [[x.copy() for x in gl] for gl in g]
            mean_h = dh0.copy()
        else:
            for l in range(len(g)):
                for i in range(3):
                    mean_w[l][i] += g[l][i]
            mean_h += dh0
    n = len(subsets)
    return [tuple(x / n for x in gl) for gl in mean_w], mean_h / n
