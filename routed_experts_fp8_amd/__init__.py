"""MI355X (gfx950) routed-expert FP8 MoE FFN layer.

The computation lives in ``libmoefp8.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/moefp8.h``); this package is its thin Python
binding plus the layer pipeline that sequences the calls.  Importing it
fails loudly if the library has not been built.
"""

from ._lib import (MoeError, fp8_block_transpose, grouped_gemm_fp8_blockscaled,
                   grouped_gemm_fp8_blockscaled_gather, quant_weight_128x128_e4m3_t, moe_sigmoid_f32,
                   moe_permute_noalloc, moe_route_permute, moe_route_permute_workspace_size,
                   grouped_gemm_fp8_combine, grouped_gemm_fp8_combine_workspace_size,
                   grouped_gemm_fp8_swiglu, moe_combine, moe_combine_backward, moe_permute,
                   moe_permute_workspace_size, moe_route, moe_route_backward, quant_act_1x128_e4m3,
                   quant_weight_128x128_e4m3, swiglu, swiglu_backward, moe_wgrad_padded_rows,
                   quant_act_128x1_grouped_e4m3, grouped_wgrad_fp8, moe_router_logits, moe_bias_update,
                   moe_probe_mfma_fp8, LIB_PATH)
from .layer import MoEBackward, MoEForward, MoEWeightGrad, quantize_weights, transpose_weights

__all__ = ["MoeError", "fp8_block_transpose", "grouped_gemm_fp8_blockscaled",
           "grouped_gemm_fp8_blockscaled_gather", "quant_weight_128x128_e4m3_t", "moe_sigmoid_f32",
           "moe_permute_noalloc", "moe_route_permute", "moe_route_permute_workspace_size",
           "grouped_gemm_fp8_combine", "grouped_gemm_fp8_combine_workspace_size",
           "grouped_gemm_fp8_swiglu", "moe_combine", "moe_permute", "moe_permute_workspace_size",
           "moe_route", "quant_act_1x128_e4m3", "quant_weight_128x128_e4m3", "swiglu",
           "moe_combine_backward", "swiglu_backward", "moe_route_backward",
           "moe_wgrad_padded_rows", "quant_act_128x1_grouped_e4m3", "grouped_wgrad_fp8",
           "moe_router_logits", "moe_bias_update", "moe_probe_mfma_fp8",
           "MoEForward", "MoEBackward", "MoEWeightGrad", "quantize_weights", "transpose_weights", "LIB_PATH"]
