"""Oracle: which t of the k chunks a sparse backward visits.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py). Shares no code with the
library's selector.

SpaCO draws t distinct chunk indices out of k without replacement (SeCO/SpaCO
review, Referee Report major comment 1, on Section 5 and Algorithm 2). The page
does not say which random generator; the reading taken is:

  * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): a 64-bit state advanced by
    the golden-ratio increment, each output mixed by two xor-shift-multiply
    rounds and a final xor-shift;
  * a partial Fisher-Yates shuffle of 0..k-1 (Knuth, TAOCP vol. 2, Algorithm P)
    stopped after t swaps, position i swapping with i + (next() mod (k - i));
  * the chosen indices returned in ascending order, 0-based.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


class SplitMix64:
    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + GOLDEN_GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def select_chunks(k: int, t: int, seed: int):
    """Ascending list of t distinct chunk indices drawn from range(k)."""
    if not (1 <= t <= k):
        raise ValueError("need 1 <= t <= k")
    gen = SplitMix64(seed)
    a = list(range(k))
    for i in range(t):
        j = i + gen.next() % (k - i)
        a[i], a[j] = a[j], a[i]
    return sorted(a[:t])
