"""Oracle: the projections on either side of one attention layer, in float64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
only the tests and the benchmark's CPU-baseline leg use it. It shares no code
with the HIP library.

What it computes. An attention layer forms its queries, keys and values from
the layer input H_in by three linear maps, Q = H_in W_q, K = H_in W_k,
V = H_in W_v (column h*d + c of a projection is element c of head h). The
StreamBP review's first major comment writes out the weight gradients the
chunked backward must produce: dW_q^(i) = H_in^(i)^T dQ^(i), and dW_k^(i) =
H_in^(:i)^T dK^(:i), dW_v^(i) = H_in^(:i)^T dV^(:i) per chunk i, whose sum over
the chunks is the dense gradient (Eq. (1)). The oracle computes the dense
quantities directly:

    dW_q = H_in^T dQ,  dW_k = H_in^T dK,  dW_v = H_in^T dV   (dQ, dK, dV as [T, H*d])
    dH_in = dQ W_q^T + dK W_k^T + dV W_v^T

with the attention part taken from oracle.attention. Matrix products are
numpy's float64 matmul (a library primitive); nothing is blocked or fused.
"""
from __future__ import annotations

import numpy as np

from . import attention


def heads_to_cols(x):
    """[B, H, T, d] -> [B, T, H*d] (column h*d + c is element c of head h)."""
    B, H, T, d = x.shape
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)).reshape(B, T, H * d))


def cols_to_heads(x, n_heads):
    """[B, T, H*d] -> [B, H, T, d]."""
    B, T, Hd = x.shape
    d = Hd // n_heads
    return np.ascontiguousarray(np.transpose(x.reshape(B, T, n_heads, d), (0, 2, 1, 3)))


def qkv_forward(h, wq, wk, wv, n_q_heads, n_kv_heads):
    """Q, K, V [B, H, T, d] from the layer input h [B, T, d_model]."""
    h = np.asarray(h, dtype=np.float64)
    q = cols_to_heads(h @ np.asarray(wq, dtype=np.float64), n_q_heads)
    k = cols_to_heads(h @ np.asarray(wk, dtype=np.float64), n_kv_heads)
    v = cols_to_heads(h @ np.asarray(wv, dtype=np.float64), n_kv_heads)
    return q, k, v


def qkv_backward(h, wq, wk, wv, dq, dk, dv):
    """Weight and input gradients of the projections (StreamBP review, major comment 1).

    dq [B, Hq, T, d], dk/dv [B, Hkv, T, d] are the gradients of Q, K, V; returns
    dW_q, dW_k, dW_v (summed over the batch) and dH_in [B, T, d_model]."""
    h = np.asarray(h, dtype=np.float64)
    gq, gk, gv = (heads_to_cols(np.asarray(x, dtype=np.float64)) for x in (dq, dk, dv))
    dwq = sum(h[b].T @ gq[b] for b in range(h.shape[0]))
    dwk = sum(h[b].T @ gk[b] for b in range(h.shape[0]))
    dwv = sum(h[b].T @ gv[b] for b in range(h.shape[0]))
    wq, wk, wv = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv))
    dh = gq @ wq.T + gk @ wk.T + gv @ wv.T
    return dwq, dwk, dwv, dh


def layer_forward(h, wq, wk, wv, n_q_heads, n_kv_heads, scale):
    """O [B, Hq, T, d] and LSE of the whole causal attention layer."""
    q, k, v = qkv_forward(h, wq, wk, wv, n_q_heads, n_kv_heads)
    o, lse = attention.forward(q, k, v, scale)
    return o, lse, (q, k, v)


def layer_backward(h, wq, wk, wv, do, n_q_heads, n_kv_heads, scale):
    """Gradients of sum(O * dO) with respect to W_q, W_k, W_v and H_in."""
    q, k, v = qkv_forward(h, wq, wk, wv, n_q_heads, n_kv_heads)
    dq, dk, dv = attention.backward(q, k, v, do, scale)
    return qkv_backward(h, wq, wk, wv, dq, dk, dv)
