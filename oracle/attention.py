"""Oracle: exact causal attention, forward and backward, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library.

What it computes. The chunk-wise methods on the pages reach exactly the dense
gradient: StreamBP's Eq. (1) writes the weight gradient as a sum over sequence
chunks of per-chunk terms (StreamBP review, "What carries the argument"), and
its Property 3.1 says chunk i's backward needs only O^(i), Q^(i), K^(:i) and
V^(:i); SeCO's gradient is reported equal to the dense one in float64 (SeCO/SpaCO
review, Referee Report summary, Appendix D). So the oracle is the plain,
unchunked definition of causal softmax attention with grouped key/value heads:

    S_rj  = scale * q_r . k_j                 visible iff j <= r (causal)
    LSE_r = ln sum_{j<=r} exp(S_rj)           (max-shifted, two passes)
    P_rj  = exp(S_rj - LSE_r)
    O_r   = sum_j P_rj v_j
    dP_rj = dO_r . v_j
    dS_rj = P_rj * (dP_rj - sum_j' P_rj' dP_rj')     softmax Jacobian
    dQ_r  = scale * sum_j dS_rj k_j
    dK_j  = scale * sum_{h in group} sum_r dS_rj q_r
    dV_j  = sum_{h in group} sum_r P_rj dO_r

q head h reads kv head h // (Hq / Hkv). The page leaves the scale out
(StreamBP review, Referee Report major comment 2: S = QK^T); it is a parameter.
The mask M^(i) is left undefined on the page (minor comment 2, Eq. (13)); the
reading here is the standard causal one at global positions.

Evaluation goes one block of query rows at a time: rows [r0, r1) against keys
[0, r1). Every row's sums still run over its whole causal prefix in one pass;
blocking only bounds memory. A subset of query rows can be requested; rows
outside it contribute nothing, which is how sampled and sparse checks are made.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


def _probs(q_blk, k_pref, scale, row_pos):
    """P and LSE for query rows at global positions ``row_pos`` over keys [0, L)."""
    s = scale * (q_blk @ k_pref.T)
    visible = np.arange(k_pref.shape[0])[None, :] <= row_pos[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    return e / den, (m + np.log(den))[:, 0]


def _row_blocks(rows, block):
    """Split a sorted array of row indices into consecutive pieces."""
    rows = np.asarray(rows, dtype=np.int64)
    for a in range(0, rows.size, block):
        yield rows[a:a + block]


def forward(q, k, v, scale, rows=None, heads=None, block=ROW_BLOCK):
    """O and LSE for query rows ``rows`` (default: all) of heads ``heads``.

    q: [B, Hq, T, d]; k, v: [B, Hkv, T, d] float64. Returns full-size arrays
    (O [B, Hq, T, d], LSE [B, Hq, T]); rows not requested are left at 0.
    """
    B, Hq, T, d = q.shape
    G = Hq // k.shape[1]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else heads
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:3], dtype=np.float64)
    for b in range(B):
        for h in heads:
            g = h // G
            for blk in _row_blocks(rows, block):
                L = int(blk[-1]) + 1
                p, l = _probs(q[b, h, blk], k[b, g, :L], scale, blk)
                o[b, h, blk] = p @ v[b, g, :L]
                lse[b, h, blk] = l
    return o, lse


def backward(q, k, v, do, scale, rows=None, heads=None, block=ROW_BLOCK):
    """dQ, dK, dV from the query rows ``rows`` of heads ``heads``.

    dK/dV collect only the contributions of the requested rows; with all rows
    and heads they are the full gradients. dQ is set on requested rows only.
    """
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else heads
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in heads:
            g = h // G
            for blk in _row_blocks(rows, block):
                L = int(blk[-1]) + 1
                kp, vp = k[b, g, :L], v[b, g, :L]
                p, _ = _probs(q[b, h, blk], kp, scale, blk)
                dp = do[b, h, blk] @ vp.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, blk] = scale * (ds @ kp)
                dk[b, g, :L] += scale * (ds.T @ q[b, h, blk])
                dv[b, g, :L] += p.T @ do[b, h, blk]
    return dq, dk, dv


def sparse_backward(q, k, v, do, scale, chunk, selected, n_chunks_total, heads=None,
                    block=ROW_BLOCK):
    """Backward with dO kept only on the selected chunks and scaled by k/t.

    The SpaCO estimator backpropagates t of the k chunks and scales the
    selected chunks' gradients by k/t (SeCO/SpaCO review, "What carries the
    argument" and Referee Report summary). With one attention layer the keys
    and values are leaves, so this is the dense backward of dO' = (k/t) * dO
    restricted to the selected rows; rows with dO' = 0 contribute exactly 0.
    """
    T = q.shape[2]
    gamma = n_chunks_total / len(selected)
    rows = np.concatenate([np.arange(i * chunk, min((i + 1) * chunk, T)) for i in sorted(selected)])
    return backward(q, k, v, gamma * do, scale, rows=rows, heads=heads, block=block)
