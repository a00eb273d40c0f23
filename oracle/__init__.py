"""CPU oracle for the EAGLE draft-and-verify round.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It is a plain, slow, obviously-correct numpy implementation written
from the pages' description of the method, and it shares no code with the HIP
library (the seeded input generators are the only common module, and they
hold none of the method's arithmetic).

Arithmetic runs in the dtype of the arrays it is given: float32 for parity
(on the same bf16-rounded values the GPU consumes, upcast), float64 for the
self-tests.

Modules:
  head    -- the draft head: fc / fusion FC, one decoder layer, LM head,
             softmax and top-k
  tree    -- chain, static (EAGLE-1) and dynamic (EAGLE-2) trees: expand,
             rerank, tree mask and position ids
  verify  -- greedy verification (longest matching root path + corrected token)
  round   -- one full draft-and-verify round built from the three above

Parity unpinned: the EAGLE-2 inverse temperature s used at the 8B shape is an
empirical constant (the mean top-1 confidence it gives is measured, not fixed
by the pages).
"""
from . import head, tree, verify, round  # noqa: F401
