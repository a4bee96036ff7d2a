"""MI355X (gfx950) library for the per-position verification pass of masked
diffusion language-model decoding.

``libdlmverify.so`` (C ABI, ``include/dlmverify.h``) holds every kernel; the
``dlmverify`` module is its Python binding with the same function names. The
library is loaded on first use, and a missing library is an error, never a
silent fallback.
"""

from .dlmverify import (  # noqa: F401
    DVError, LIB_PATH, RULES, STAT_FIELDS, CORE_FIELDS, DV_LOGITS_NEG_INF, load_library, dv_verify_workspace_bytes, dv_verify_rows, VerifyPlan, Prepared, prepare_seed_score, prepare_select_topk, prepare_seed_select, prepare_decide, prepare_decide_seed_select, prepare_seed_select_decide, prepare_influence_drift, dv_verify_rows_noalloc, DV_NOALLOC_SCRATCH_BYTES, dv_decide,
    dv_seed_score, dv_select_topk, dv_seed_select, dv_decide_seed_select, dv_seed_select_decide, dv_tree_accept, dv_influence_drift_workspace_bytes, dv_influence_drift,
    dv_dual_view_attention, dv_debug_hash, dv_debug_noise, DEBUG_NOISE_MODES, dv_debug_read_probe, dv_status_str, dv_last_error, dv_version,
    DV_NONE, DV_KEEP, DV_REPLACE, DV_REMASK,
)
