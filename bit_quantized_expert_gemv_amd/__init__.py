"""Quantised MoE expert layer for AMD MI355X (gfx950): router GEMV, softmax top-K, 4-bit and
2-bit group-affine dequantised expert GEMVs, SwiGLU, and a combine with a gated shared expert
plus the residual.

The compute lives in ``libbqmoe.so`` (C ABI in ``include/moe.h``). This package is its thin
Python binding, with the same names as the C entry points.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    MOE_EHIP,
    MOE_EINVAL,
    MOE_ENOSPC,
    MOE_EUNSUPPORTED,
    MOE_MAX_EXPERTS,
    MOE_MAX_TOP_K,
    MOE_OK,
    MOE_PREFILL_MIN_TOKENS,
    MOE_ROUTER_BATCH_MIN_TOKENS,
    MOE_ROUTER_CERTIFIED_MIN_TOKENS,
    MOE_FLAG_DEQUANT_LITERAL,
    MOE_FLAG_DEQUANT_NAIVE,
    MOE_NOALLOC_SCRATCH_BYTES,
    SIGNATURES,
    MoeError,
    lib,
    make_layer,
    moe_blob_bytes,
    moe_combine,
    moe_dequant,
    moe_expert_arrays_t,
    moe_expert_ffn,
    moe_expert_ffn_checked,
    moe_last_error,
    moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_layer_forward_timed,
    moe_layer_t,
    moe_pack_expert,
    moe_pack_expert_device,
    moe_router,
    moe_router_approx_logits,
    moe_stack_forward,
    moe_stack_workspace_bytes,
    moe_strerror,
    moe_workspace_bytes,
    ptr,
    stream_handle,
)
