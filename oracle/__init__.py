"""fp64 CPU oracle for sparse bidirectional attention — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct statement of what the GPU
library computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library itself never does, and this
package imports nothing from the library.  It shares no code with the GPU
path: the only common module is the seeded input generator (`workloads`),
which holds none of the method's arithmetic.

Everything is numpy in float64.  bf16 inputs are decoded exactly to float64.

Modules
  attention : dense, token-masked, block-sparse and column-sparse softmax
              attention (the definition, with its log-sum-exp).
  select    : block mean-pooling, pooled scores and their softmax mass,
              the exact block mass from the full attention, top-k and
              mass-with-global-cap block selection to CSR, exact column
              scores and column top-k.
  losa      : LoSA-style partial attention for block-wise diffusion: the
              query-change locality score, the Active set, per-query page
              selection, the per-kv-head page union and the attention of
              Active rows over (union pages + block) with Stable rows kept.
  schedule  : the per-step action table (warm-up, selection, reuse, refresh,
              probes), the overlap of two block patterns and the probe's
              adoption rule, and a whole-schedule runner for small shapes.

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to
brute force, closed forms, library routines or invariants; no function is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    block_sparse_attention,
    block_token_mask,
    column_sparse_attention,
    column_token_mask,
    decode_bf16,
    default_scale,
    dense_attention,
    head_group,
    masked_attention,
)
from .select import (  # noqa: F401
    column_scores,
    count_from_fraction,
    exact_block_mass,
    pool_blocks,
    pooled_mass,
    pooled_scores,
    rank_order,
    select_columns,
    select_mass_cap,
    select_topk,
)
from .schedule import (  # noqa: F401
    ACTIONS,
    mask_overlap,
    overlap_ratio,
    probe_adopts,
    run_schedule,
    schedule_actions,
    select_steps,
)
from .losa import (  # noqa: F401
    block_attention,
    locality_scores,
    losa_attention,
    losa_dense,
    losa_step,
    page_scores,
    pool_pages,
    select_active,
    select_pages,
    union_pages,
    union_token_mask,
)
