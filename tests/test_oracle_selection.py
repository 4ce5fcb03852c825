"""Pins for the oracle's chunk selector (SplitMix64 + partial Fisher-Yates)."""
import collections
import os

from oracle.selection import SplitMix64, select_chunks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_splitmix64_published_outputs():
    gen = SplitMix64(0)
    for want in _lines("splitmix64_seed0.txt"):
        assert gen.next() == int(want, 16)


def test_hand_traced_selections():
    for ln in _lines("selection_hand_traced.txt"):
        head, tail = ln.split(":")
        k, t, seed = map(int, head.split())
        assert select_chunks(k, t, seed) == [int(x) for x in tail.split()]


def test_selection_properties():
    for k in (1, 2, 7, 64):
        for t in sorted({1, max(1, k // 8), k // 2 or 1, k}):
            for seed in range(5):
                s = select_chunks(k, t, seed)
                assert len(s) == t and len(set(s)) == t
                assert s == sorted(s) and 0 <= s[0] and s[-1] < k
    assert select_chunks(9, 9, 123) == list(range(9))


def test_selection_inclusion_frequency():
    # sanity only: each chunk is kept with probability t/k under uniform subsets
    k, t, n = 16, 4, 4000
    cnt = collections.Counter()
    for seed in range(n):
        cnt.update(select_chunks(k, t, seed))
    for c in range(k):
        assert abs(cnt[c] / n - t / k) < 0.03
