"""DropKV eviction scoring on AMD Instinct MI355X (gfx950).

The scoring runs in hand-written HIP kernels inside libdropkv.so, reached
through a C ABI (include/dropkv.h); `binding` marshals torch GPU tensors to
it. `synth` draws the seeded synthetic inputs. Importing the package does not
load the library; the first call does, and fails loudly if it is not built.
"""

from .binding import (  # noqa: F401
    BF16, F32, FLAG_GENERIC, FLAG_STAGE_LOG, STATUS_BAD_INDEX, STATUS_NONFINITE, STATUS_SINGULAR,
    STATUS_NEGATIVE, DecodeScorer, DropKVError, DropKVNegativeScoreError,
    DropKVInvalidError, DropKVNonFiniteError, DropKVNotBuiltError, DropKVSingularError, LIB_PATH,
    compact, compact_kept, load_library, pass1_stats, prefill_attention, raw_scores, row_stats, score, score_ex, score_keep_ex, score_from_stats, select,
    stage_log, stage_times,
    uses_mfma,
    version,
    workspace_bytes,
)

__all__ = [
    "score", "score_ex", "score_keep_ex", "score_from_stats", "raw_scores", "row_stats", "pass1_stats", "select", "compact", "compact_kept",
    "DecodeScorer", "DropKVNegativeScoreError", "STATUS_NEGATIVE", "prefill_attention",
    "stage_times", "stage_log",
    "workspace_bytes",
    "uses_mfma",
    "load_library", "version", "DropKVError", "DropKVInvalidError", "DropKVSingularError",
    "DropKVNonFiniteError", "DropKVNotBuiltError", "BF16", "F32", "FLAG_GENERIC", "FLAG_STAGE_LOG",
    "STATUS_SINGULAR", "STATUS_NONFINITE", "STATUS_BAD_INDEX", "LIB_PATH",
]
