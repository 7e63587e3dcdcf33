"""MI355X-native single-GPU MoE expert layer: route -> permute -> m-grouped SwiGLU -> combine.

The compute runs in hand-written HIP kernels (libmoe_mi355x.so, C ABI in
include/moe.h); this package only marshals torch tensors into those calls.
"""
from ._binding import (LIB_PATH, MOE_BF16, MOE_F32, MOE_MX_KSTEPS, MOE_MX_ROWS, SIGNATURES, MoEError, grouped_workspace,
                       lib, moe_capacity, moe_combine, moe_combine_backward,
                       moe_grouped_dgrad_fc1, moe_grouped_dgrad_swiglu, moe_grouped_fc1_swiglu,
                       moe_grouped_fc2, moe_grouped_swiglu, moe_grouped_wgrad,
                       moe_grouped_fc1_swiglu_mxfp8, moe_grouped_swiglu_masked,
                       moe_grouped_workspace_bytes, moe_permute, moe_permute_masked,
                       moe_permute_noalloc,
                       moe_permute_mxfp8, moe_permute_workspace_bytes, moe_quantize_mxfp8,
                       moe_round_bf16, moe_route, moe_status_str)
from .layer import (DenseRows, MxWeights, SharedExperts, moe_layer, moe_layer_backward,
                    moe_layer_masked, moe_layer_mxfp8)

__all__ = [
    "LIB_PATH", "MOE_BF16", "MOE_F32", "MOE_MX_KSTEPS", "MOE_MX_ROWS", "SIGNATURES", "MoEError", "grouped_workspace", "lib",
    "moe_capacity", "moe_combine", "moe_combine_backward", "moe_grouped_dgrad_fc1",
    "moe_grouped_dgrad_swiglu", "moe_grouped_fc1_swiglu", "moe_grouped_fc2", "moe_grouped_swiglu",
    "moe_grouped_wgrad", "moe_grouped_swiglu_masked", "moe_grouped_workspace_bytes",
    "moe_grouped_fc1_swiglu_mxfp8", "moe_permute", "moe_permute_masked", "moe_permute_mxfp8",
    "moe_permute_noalloc",
    "moe_quantize_mxfp8", "moe_round_bf16",
    "moe_permute_workspace_bytes", "moe_route", "moe_status_str", "DenseRows", "SharedExperts",
    "moe_layer", "moe_layer_backward", "moe_layer_masked", "moe_layer_mxfp8", "MxWeights",
]
