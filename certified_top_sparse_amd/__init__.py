"""certified_top_sparse_amd -- certified Top-k attention truncation on MI355X.

The compute lives in libctopk.so (hand-written HIP kernels for gfx950, C ABI
declared in include/ctopk.h).  This package holds the kernels' sources
(csrc/), the in-tree build script (build.py) and a ctypes binding (ctopk.py)
whose functions carry the C names.
"""
from .ctopk import (  # noqa: F401
    CTOPK_BF16, CTOPK_F32, CTOPK_FLAG_BOUND, CTOPK_PLAN_DECODE, CTOPK_PLAN_DECODE_BOUND,
    CTOPK_PLAN_DECODE_FUSED, CTOPK_PLAN_DECODE_OVERLAP, CTOPK_PLAN_ENCODER,
    CtopkArgs, CtopkError, CtopkK4Args, EXPORTED, LIB_PATH, ctopk_candidates_k4, ctopk_certify,
    ctopk_certify_ex, ctopk_certify_logits, ctopk_certify_noalloc, CTOPK_NOALLOC_SCRATCH_BYTES, ctopk_last_error_string,
    ctopk_logits_workspace_bytes, ctopk_plan, ctopk_record_kernel_events, ctopk_validate,
    ctopk_k4_workspace_bytes, ctopk_quantize_k4, ctopk_validate_k4, ctopk_version,
    ctopk_workspace_bytes, make_k4_args,
    default_scale, load, make_args,
)
