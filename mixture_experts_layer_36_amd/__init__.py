"""MI355X (gfx950) MoE layer forward: HIP kernels behind a C ABI (include/moe.h).

The Python surface mirrors the C entry points one to one and only marshals
arguments; see _lib.py.
"""
from ._lib import (  # noqa: F401
    BF16, EXPORTS, F32, FP8_E4M3, LIB_PATH, MOE_ERR_DEVICE, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE, MOE_OK, SIGMOID, SOFTMAX, STAGE_DISPATCH, STAGE_FFN, STAGE_LAYER,
    STAGE_ROUTE, TRACE_EVENTS, TRACE_STAGES, Desc, MoeError, capacity_slots, combine, dispatch,
    dispatch_noalloc, NOALLOC_SCRATCH_BYTES,
    fp8_payload_bytes, fp8_payload_views, fp8_scale_stride, fp8_scales_offset, grouped_ffn, layer_forward,
    layer_rows, pack_weights, W_KBLOCKED, W_ROWMAJOR, route_candidates, dispatch_reroute,
    loaded_path, route, validate, workspace, workspace_size,
)
