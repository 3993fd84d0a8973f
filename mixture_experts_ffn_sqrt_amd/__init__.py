"""MI355X-native (gfx950) single-GPU Mixture-of-Experts FFN layer.

The layer runs in hand-written HIP kernels behind a C ABI (include/moe.h,
libmoe.so); `binding` is its thin Python wrapper and `synth` draws the seeded
synthetic inputs.
"""
from .binding import (  # noqa: F401
    EXPORTS, MOE_BF16, MOE_F32, MOE_ROUTE_HASH, MOE_ROUTE_LEARNED, MOE_SCORE_SIGMOID,
    MOE_SCORE_SOFTMAX, MOE_SCORE_SQRTSOFTPLUS, MoeConfig, MoeError, MoELayer, load_library,
    make_config, moe_combine, moe_expert_down, moe_expert_down_fp8, moe_expert_ffn, moe_expert_up,
    moe_expert_up_fp8, moe_forward, moe_forward_fp8, moe_forward_noalloc, moe_permute,
    moe_quantize_fp8_blocks,
    moe_quantize_fp8_rows, moe_route, moe_strerror, moe_workspace_size, quantize_fp8_weights,
    moe_quantize_mxfp4, moe_expert_up_mxfp4, moe_expert_down_mxfp4, moe_forward_mxfp4,
    quantize_mxfp4_weights)
