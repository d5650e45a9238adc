"""CPU fp64 oracle for masked softmax attention (test infrastructure only).

This package is the correctness reference for the HIP path.  Only the tests,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
library never does, and it imports nothing from the library.

Contents
  masks      closed-form mask predicates allowed(i, j) for the 12 static
             patterns, the two block-sparse patterns and ring-step masks
  attention  plain softmax attention forward / backward in fp64
  tiles      brute-force tile classification (EMPTY / FULL / PARTIAL),
             visit lists and exact pair counts from a dense mask
  merge      log-sum-exp merge of partial attention results
  blockscore block importance scores from mean-pooled Q and K (dynamic
             block-sparse masks)

Source: "Long-Context Attention Benchmark: From Kernel Efficiency to
Distributed Context Parallelism" (LongCA-bench) and its summaries.  The pages
define the problem (standard quadratic softmax attention, section 1; the naive
step-by-step baseline that supports any mask, section 3.1 and the notes' key
design 2) but print no formulas, so the oracle is the textbook definition
written out.  Where the pages leave a mask undefined the reading used is
stated beside the predicate.

Parity unpinned against the pages themselves: they print no numeric result
for this computation.  The oracle is pinned instead by brute force, by
closed forms, by a library routine on special cases and by invariants (see
tests/test_oracle_*.py).  Two mask definitions are this build's readings and
are parity unpinned as to identity: PREFIX_LM_DOCUMENT (the unnamed sixth
heterogeneous mask) and CAUSAL_BLOCKWISE (read literally).
"""
from . import masks, attention, tiles, merge, blockscore  # noqa: F401
