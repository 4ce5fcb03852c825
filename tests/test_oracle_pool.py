"""The thread-pooled oracle evaluation used by the full-size GPU checks equals
direct calls of oracle.attention (it only splits heads and row ranges and sums
the pieces' dK/dV), so the full-size checks compare against the oracle itself."""
import numpy as np

import oracle_pool as P
from oracle import attention as A


def test_pooled_equals_direct():
    rng = np.random.default_rng(1)
    T, Hq, Hkv, d, scale = 700, 4, 2, 16, 0.3
    q, do = rng.standard_normal((2, 1, Hq, T, d))
    k, v = rng.standard_normal((2, 1, Hkv, T, d))
    dq, dk, dv = A.backward(q, k, v, do, scale)
    o, lse = A.forward(q, k, v, scale)
    for g in range(Hkv):
        a, b, c = P.group_backward(q, k, v, do, scale, g)
        assert np.abs(a - dq[0, 2 * g:2 * g + 2]).max() < 1e-13
        assert np.abs(b - dk[0, g]).max() < 1e-13 and np.abs(c - dv[0, g]).max() < 1e-13
    rows = np.sort(rng.choice(T, 200, replace=False))
    dq2, dk2, dv2 = A.backward(q, k, v, do, scale, rows=rows, heads=[2, 3])
    a, b, c = P.group_backward(q, k, v, do, scale, 1, rows=rows)
    assert np.abs(a - dq2[0, 2:4]).max() < 1e-13
    assert np.abs(b - dk2[0, 1]).max() < 1e-13 and np.abs(c - dv2[0, 1]).max() < 1e-13
    for h in range(Hq):
        a, b = P.head_forward(q, k, v, scale, h)
        assert np.abs(a - o[0, h]).max() < 1e-13 and np.abs(b - lse[0, h]).max() < 1e-13


def test_row_ranges_cover_rows_once():
    rows = np.arange(1000)
    parts = P.row_ranges(rows, 7)
    assert np.array_equal(np.concatenate(parts), rows)
    assert len(parts) == 7
