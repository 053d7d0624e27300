"""CPU oracle for TriangleMix triangle-attention prefill.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the GPU library (``static_triangle_sparse_amd``) and neither side
imports the other; both read their inputs from the seeded generators in
``synth``.

What it computes (all in float64, from the exact bf16 input values):

* ``mask``      -- the static mask predicate of one attention layer (full
                   causal, or triangle = sink keys + diagonal window + last
                   query rows, middle skipped) and the kept-tile list it
                   induces on a (block_q x block_k) grid, by brute force.
* ``attention`` -- masked softmax attention (output rows and per-row
                   log-sum-exp) as the plain definition, one BLAS product
                   per row block over the gathered kept keys.
* ``brute``     -- the same quantities with pure-Python loops and
                   ``math.fsum``, for tiny inputs only.
* ``dynamic``   -- dynamic block-sparse tile selection for the dense layers
                   (probe queries against pooled keys, max-based threshold;
                   FlashPrefill page, sections 2.1-2.3) and attention over an
                   explicit per-head tile list.
* ``tiers``     -- triangle attention with fp8 (e4m3) scores on tiles past a
                   per-head diagonal-distance boundary (TriAttention page),
                   with its e4m3 rounding and block scales.

Sources (the pages this method is described on):
  * "TriangleMix" blog post (PaperWeekly / news.fishai.com.cn), sections
    "介绍" (Introduction) and "缘由" (Origin): shallow layers dense, deep
    layers use the triangle pattern; the "Middle Q-K" part is removed.
  * "Yang Yuqing von Microsoft Research" (36kr), technical-motivation
    paragraphs: only the streaming region (the beginning part) and the final
    "Last Q-K" aggregation region are kept; complexity falls to O(N).

Every function here is pinned by tests in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_dynamic.py`` and ``tests/test_oracle_tiers.py``
(brute force, closed forms, library attention on the special cases that
reduce to it, and hand-derived tile grids); none is "parity unpinned".
"""
from . import mask, attention, brute, dynamic, tiers  # noqa: F401
