"""Oracle: a plain, slow, fp64 CPU definition of the speculative-decoding
verify step, used only to check the GPU path.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call anything here; the
product path (the C-ABI library and its Python binding) never does, and
shares no code, table or constant with it.

Modules:
  philox  -- Philox4x32-10 from its published definition (Salmon et al.,
             SC'11), and the two verify uniforms per (seed, sequence, position).
  verify  -- LM-head logits, greedy acceptance, speculative sampling with
             residual / bonus draw, decision margins, the closed-form
             expected tokens per verify pass, and both rules on packed
             batches with per-sequence draft counts.
  tree    -- greedy verification of a draft tree (longest accepted path).
  ngram   -- the prompt-lookup drafter (most recent earlier occurrence of
             the longest matching suffix n-gram).

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to
something other than itself: published Philox known-answer blocks and an
independent library implementation, exact rational arithmetic for the
logits, brute force over every draft sequence for greedy decoding,
chi-square tests of the sampled output against the target distribution, the
closed form for the expected tokens per pass, the residual identity, and
(for packed batches) reduction to the dense rule sequence by sequence, and
(for trees) reduction to the linear rule on chains plus brute force against
target-only greedy decoding; the n-gram drafter by an independent string
search and hand-worked sequences.
"""
from .philox import philox4x32_10, uniform24, verify_uniforms  # noqa: F401
from .verify import (  # noqa: F401
    GreedyResult, SampleProbs, SampleResult, accept_greedy, accept_greedy_ragged, accept_ratio, accept_sample,
    accept_sample_probs, accept_sample_ragged, accept_sample_rounds, sample_probs, expected_tokens, expected_tokens_positional, inverse_cdf, lm_head_logits,
    ragged_sequences, softmax, widen_bf16,
)
from .tree import TreeResult, tree_accept_greedy  # noqa: F401,E402
from .ngram import ngram_propose, ngram_propose_one, trailing_runs  # noqa: F401,E402
