"""Routed Mixture-of-Experts FFN with group-quantised experts on MI355X (gfx950).

The compute lives in libmoe.so (HIP kernels behind the C ABI of
include/moe.h). This package holds its ctypes binding, the build script and
the byte / op accounting used to price a run against the chip's roofline.
"""
from ._lib import (  # noqa: F401
    ACT_MODES, FORMATS, ROUTERS, STAGES, MOE_STAGE_COUNT, WS_SECTIONS,
    MOE_ACT_F32, MOE_ACT_Q8_0, MOE_W_INT4_G32, MOE_W_INT8_G32, MOE_W_INT2_G32, MOE_W_INT4_ROW, MOE_W_INT8_ROW,
    MOE_W_INT2_ROW,
    MOE_ROUTER_SOFTMAX_TOPK, MOE_ROUTER_SIGMOID_NOAUX_TC,
    MoeError, QuantExperts, RouterParams, Experts,
    load, exported_names, router_params, with_top_p, quantize_experts, workspace,
    moe_workspace_size, moe_quantize_weights, moe_quantize_q8_0, moe_route, moe_dispatch,
    moe_expert_ffn, moe_debug_q8_expert_ffn, moe_debug_workspace_sections, moe_combine, moe_layer_forward,
    moe_layer_forward_noalloc, moe_layer_forward_timed, MOE_NOALLOC_SCRATCH_BYTES,
    moe_block_forward, moe_calib_stream_read, moe_calib_prefill_mix,
    moe_status_string, moe_last_error_detail,
)
