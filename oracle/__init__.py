"""fp64 CPU oracle for DropKV eviction scoring (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never uses it and must fail loudly when
its own extension is missing rather than fall back here.
"""
from .dropkv_oracle import (  # noqa: F401
    SINGULAR_REST_MASS, SingularRow, NonFiniteInput, bf16_bits_to_f64, as_f64,
    window_positions, group_rows, row_attention, head_row_stats, perturbation_sq,
    head_scores, maxpool1d_same, protect_window, evict_smallest, check_args,
    dropkv_oracle, compact_cache,
)
from .joint import joint_objective, approx_ratio  # noqa: F401
from .decode import decode_init, decode_step, decode_scratch, decode_select  # noqa: F401
from .prefill import prefill_outputs  # noqa: F401
