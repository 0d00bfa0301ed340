"""IKBO (In-Kernel Broadcast Optimization) target attention for MI355X.

The compute lives in libikbo.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/ikbo.h).  This package holds the sources, the build script and
a ctypes binding whose functions carry the C entry points' names.
"""

from .ikbo import (  # noqa: F401
    IKBO_DTYPE_BF16,
    IKBO_DTYPE_F32,
    IKBO_ERR_BAD_MAPPING,
    IKBO_ERR_BAD_OFFSETS,
    IKBO_ERR_HIP,
    IKBO_ERR_INVALID_ARG,
    IKBO_ERR_NOMEM,
    IKBO_ERR_UNSUPPORTED,
    IKBO_OK,
    SIGNATURES,
    IkboError,
    ikbo_attn_fwd,
    ikbo_attn_fwd_ex,
    ikbo_attn_fwd_materialized,
    ikbo_attn_fwd_planned,
    ikbo_group_csr,
    ikbo_last_error,
    ikbo_attn_bwd,
    ikbo_bwd_create,
    ikbo_bwd_destroy,
    ikbo_bwd_info,
    ikbo_bwd_timing,
    ikbo_bwd_timing_read,
    ikbo_lce_create,
    ikbo_lce_destroy,
    ikbo_lce_errors,
    ikbo_lce_fwd,
    ikbo_lce_timing,
    ikbo_lce_timing_read,
    ikbo_plan_build,
    ikbo_plan_create,
    ikbo_plan_destroy,
    ikbo_plan_info,
    ikbo_plan_timing,
    ikbo_plan_trace,
    ikbo_plan_trace_read,
    ikbo_plan_timing_read,
    ikbo_self_target_fwd,
    ikbo_version,
    load_library,
)
