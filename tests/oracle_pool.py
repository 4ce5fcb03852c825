"""Thread-pooled evaluation of the float64 oracle for full-size parity checks.

Test infrastructure. Every number still comes from oracle.attention: the work
of one kv group is cut into (q head, contiguous range of query rows) pieces,
each evaluated by oracle.attention.forward / backward on that head alone, and
the pieces' dK/dV are summed (float64; the order of that sum is the only
difference from a single call, a rounding-level change). numpy releases the
GIL inside its large array operations and BLAS, so a thread pool runs the
pieces in parallel; BLAS itself is held to one thread per piece.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import attention as A


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def row_ranges(rows: np.ndarray, pieces: int):
    """Split sorted query rows into contiguous runs with about equal causal work
    (a row r costs r + 1 visible keys)."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return []
    cost = np.cumsum(rows + 1, dtype=np.float64)
    bounds = np.searchsorted(cost, cost[-1] * np.arange(1, pieces) / pieces)
    out, a = [], 0
    for b in list(bounds) + [rows.size]:
        if b > a:
            out.append(rows[a:b])
            a = b
    return out


def _pool_map(fn, tasks):
    """Yield fn(task) in task order; results are consumed as they arrive."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        with ThreadPoolExecutor(_workers()) as ex:
            yield from ex.map(fn, tasks)


def group_backward(q, k, v, do, scale, group, rows=None):
    """dQ of the group's q heads and dK, dV of kv head ``group`` (batch entry 0),
    from query rows ``rows`` (default all). Returns (dq [G, T, d], dk [T, d], dv [T, d])."""
    Hq, T = q.shape[1], q.shape[2]
    G = Hq // k.shape[1]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    pieces = max(1, math.ceil(2 * _workers() / G))
    tasks = [(h, r) for h in range(group * G, (group + 1) * G) for r in row_ranges(rows, pieces)]
    kg, vg = k[:1, group:group + 1], v[:1, group:group + 1]

    def run(task):
        h, r = task
        return h, A.backward(q[:1, h:h + 1], kg, vg, do[:1, h:h + 1], scale, rows=r)

    dq = np.zeros((G, T, q.shape[3]))
    dk = np.zeros((T, q.shape[3]))
    dv = np.zeros((T, q.shape[3]))
    for h, (a, b, c) in _pool_map(run, tasks):
        dq[h - group * G] += a[0, 0]
        dk += b[0, 0]
        dv += c[0, 0]
    return dq, dk, dv


def head_forward(q, k, v, scale, head):
    """O [T, d] and LSE [T] of one q head (batch entry 0) over every row."""
    Hq, T = q.shape[1], q.shape[2]
    g = head // (Hq // k.shape[1])
    tasks = row_ranges(np.arange(T), 2 * _workers())

    def run(r):
        return A.forward(q[:1, head:head + 1], k[:1, g:g + 1], v[:1, g:g + 1], scale, rows=r)

    o = np.zeros((T, q.shape[3]))
    lse = np.zeros(T)
    for r, (a, b) in zip(tasks, _pool_map(run, tasks)):
        o[r] = a[0, 0, r]
        lse[r] = b[0, 0, r]
    return o, lse
