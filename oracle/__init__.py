"""Oracle for chunked causal attention: plain float64 CPU definitions.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import this package. The HIP library neither imports nor
calls it, and the two share no code.

Pins (tests/test_oracle_*.py): central finite differences, float64
torch.autograd on the naive masked-softmax formula, closed forms (K = 0,
T = 1), invariants (row sums, shift and scale invariance, GQA vs repeated
heads), the chunk-sum identity and exhaustive sparse-subset averaging. The
selector is pinned by SplitMix64's published first outputs for seed 0 and a
hand-traced shuffle. No function here is "parity unpinned".
"""
from . import attention, selection  # noqa: F401
