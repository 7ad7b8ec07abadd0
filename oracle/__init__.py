"""fp64 CPU oracle for the Fast-dLLM block-decoding hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  The HIP library
never calls it and must fail loudly when its own extension is missing.

It shares no code with the HIP path: no kernels, headers, helpers, tables or
pre/post-processing.  Inputs come from ``workloads`` (seeded generators that
hold none of the method's arithmetic).

Parity status of each function (pins live in tests/test_oracle_*.py):

* ``fresh_range``       pinned (closed form per mode, hand-checked cases)
* ``attn_ref``          pinned (SDPA in float64, closed forms, hand-computed
                        golden fixture, post-refresh identity, nested-mode
                        equalities, GQA==MHA, batch permutation)
* ``row_confidence``    pinned (scipy softmax, sigmoid identity, calibrated
                        recipe, hand-computed golden fixture)
* ``unmask_ref``        pinned (brute force over all masks for tiny blocks,
                        tau>=1 -> one token, tau below all -> whole block,
                        monotonicity, hand-computed golden fixture)
* ``refresh_ref``       pinned (bit-exact copy, sentinel, idempotence, subset)
* ``decode_block_ref``  pinned (step counts 1..m, tau>=1 -> m steps)
* ``unmask_topk_ref``   pinned (k >= m -> whole block, k = 1 -> the
                        threshold rule's single-best fallback, top-k == the
                        threshold rule at a threshold between the k-th and
                        (k+1)-th confidence, brute-force ordering over all
                        masks of a small block, unread rows)
* ``tokens_per_step``   pinned (the pages' own flag settings)
* ``decode_block_topk_ref`` pinned (ceil(m / k) steps of k tokens)
* ``lmhead_logits_ref`` pinned (brute-force dot products with exact sums,
                        one-hot projection closed form, exact integer
                        products on the grid inputs)
* ``lmhead_unmask_ref`` pinned (equals the pinned unmask rules applied to
                        brute-force logits; the logits' argmax on planted rows)
* model-level quality (accuracy, real staleness drift, Theorem 1):
  parity unpinned -- needs trained weights and datasets, out of scope.
"""
from .fdllm_oracle import (  # noqa: F401
    fresh_range,
    attn_ref,
    row_confidence,
    unmask_ref,
    UnmaskResult,
    refresh_ref,
    decode_block_ref,
    unmask_topk_ref,
    tokens_per_step,
    decode_block_topk_ref,
    lmhead_logits_ref,
    lmhead_unmask_ref,
    NEAR_TIE,
)
