"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so neither the oracle nor the HIP library depends on the
other through it.

Workload recipe: the pages measure on PG-19 test-set prefixes with trained
models; neither is available, and the hot path's speed depends only on the
shapes, so seeded Gaussian inputs of the pages' model shapes stand in for them.

* K, V and Q entries are N(0, 1) float32 draws rounded to bfloat16
  (round-to-nearest-even). The 1.5B-class keys carry one U(0.5, 2) scale per
  (KV head, channel).
* Logits are N(0, sigma^2) float32 with sigma = 2 by default; window ids are
  uniform over the vocabulary.
* Acceptance inputs: uniform target tokens over a small vocabulary; each
  draft token copies its parent's target token with probability p_match
  (default 1/2), so paths of every length occur.
* N-gram windows: uniform tokens with a few fixed 4-token phrases copied in
  at random positions (repeated phrases, as generated text has).
* Parity inputs use NumPy's PCG64 (``default_rng(seed)``).
"""

from .inputs import (
    bf16_round,
    attention_inputs,
    penalty_inputs,
    CONFIGS,
    tree_parent,
    random_parent,
    accept_inputs,
    ngram_window,
)

__all__ = ["bf16_round", "attention_inputs", "penalty_inputs", "CONFIGS", "tree_parent", "random_parent",
           "accept_inputs", "ngram_window"]
