"""Plain float64 CPU oracle for the TokenSwift per-step hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP library (no kernels,
headers, helpers, tables or constant generators); inputs reach both sides from
the seeded generators in ``synth``, which hold none of the method's arithmetic.

Every function states the definition it writes out and cites the passage it
follows. Page names used in the citations:

* "TokenSwift summary" -- the paperlayer.ai source-linked summary of
  *TokenSwift: Lossless Acceleration of Ultra Long Sequence Generation*
  (arXiv 2502.18890v2); sections are the paper's own numbers.
* "TokenSwift reproducibility checklist" -- the acmrep2026 page on the same
  paper (its Table 11 lists the inference hyper-parameters).

Every part reaches an exactly defined result (the method is lossless), so
each oracle is that definition written out in float64, vectorised only with
library primitives (matrix products, sorts, cumulative sums). Where the pages
are silent the reading taken is stated next to the code.

Parity status: every public function is pinned by ``tests/test_oracle_*.py``
against library routines, closed forms and brute force; none is "parity
unpinned".
"""

from .common import bf16_to_f64, ancestor_sets
from .attention import verify_attention, draft_attention
from .select import partial_kv_select, SelectResult
from .penalty import penalty_sample, PenaltyResult, eta_sample, EtaResult
from .accept import accept_path, kv_commit
from .ngram import ngram_candidates, ngram_tree, splitmix64

__all__ = [
    "bf16_to_f64",
    "ancestor_sets",
    "verify_attention",
    "draft_attention",
    "partial_kv_select",
    "SelectResult",
    "penalty_sample",
    "PenaltyResult",
    "eta_sample",
    "EtaResult",
    "accept_path",
    "kv_commit",
    "ngram_candidates",
    "ngram_tree",
    "splitmix64",
]
