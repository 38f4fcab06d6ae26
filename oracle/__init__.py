"""Slow, plain fp64 CPU oracle for per-head heterogeneous block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``head_heterogeneous_block_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.  The only
thing both consume is the seeded synthetic input produced by
``head_heterogeneous_block_amd.workloads`` (random draws, no method arithmetic).
"""

from .block_sparse import (  # noqa: F401
    to_f64,
    pool_blocks,
    budget_blocks,
    forced_blocks,
    select_row,
    prefill_block_scores,
    select_blocks_prefill,
    attention_prefill_gather,
    attention_prefill_dense_masked,
    prefill_tile_loads,
    attended_flops_prefill,
    decode_select,
    decode_attention,
    decode_attention_dense,
    lpt_schedule,
    brute_force_makespan,
)
from .calibration import (  # noqa: F401
    block_attention_mass,
    row_recovery,
    head_recovery,
    recovery_table,
    needed_ratio,
    maxmin_shift,
    brute_force_maxmin,
    output_deviation,
    deviation_table,
    needed_ratio_deviation,
)
