"""MI355X (gfx950) routed mixture-of-experts feed-forward layer.

The compute path is libmoe.so (hand-written HIP kernels behind a C ABI,
include/moe.h); this package is its thin Python binding.
"""
from ._lib import (EXPORTS, LIB_PATH, OP_GROUPED_FFN, OP_GROUPED_FFN_NVFP4, OP_PERMUTE, OP_REFILL_SCORE,
                   OP_ROUTE, OP_ROUTE_PERMUTE, OUT_BF16, OUT_F32, LayerCall, MoeError, Workspace,
                   awq_to_output_major, combine, grouped_ffn, grouped_ffn_noalloc, layer, layer_workspace_bytes,
                   lib, moe_layer, noalloc_max_bytes, nvfp4_quantize, permute, prune_slice, refill_finalize,
                   refill_score, route, route_permute, router_norm_keep, workspace_bytes)
from .calibration import RefillCalibration

__all__ = ["EXPORTS", "LIB_PATH", "OP_GROUPED_FFN", "OP_GROUPED_FFN_NVFP4", "OP_PERMUTE", "OP_REFILL_SCORE",
           "OP_ROUTE", "OP_ROUTE_PERMUTE", "OUT_BF16", "OUT_F32", "LayerCall", "MoeError", "Workspace",
           "awq_to_output_major", "combine", "grouped_ffn", "grouped_ffn_noalloc", "layer",
           "layer_workspace_bytes", "lib", "moe_layer", "noalloc_max_bytes", "nvfp4_quantize", "permute",
           "prune_slice", "refill_finalize", "refill_score", "route", "route_permute", "router_norm_keep",
           "workspace_bytes", "RefillCalibration"]
