"""Routed-expert Mixture-of-Experts forward path for one AMD Instinct MI355X (gfx950).

The layer runs as five calls of the HIP library ``libmoe_mi355x.so`` (C ABI in
``include/moe_mi355x.h``): top-k routing, an atomic-free permute into a padded
expert-grouped layout, a grouped gate/up GEMM with fused SwiGLU, a grouped
down GEMM and an fp32 score-weighted gather-sum.  ``_lib`` binds them; torch
only provides device memory and streams.
"""
from .build import library_path  # noqa: F401

_API = ("route_topk", "permute", "grouped_glu_gemm", "grouped_down_gemm", "combine",
        "moe_forward", "MoELayer", "MoEError", "Layout", "padded_rows_max",
        "permute_workspace_size", "load", "grouped_glu_gemm_gather", "FP8Weights", "quantize_fp8",
        "grouped_glu_gemm_fp8w", "grouped_glu_gemm_gather_fp8w", "grouped_down_gemm_fp8w",
        "grouped_gemm", "grouped_gemm_swiglu_backward", "grouped_glu_gemm_clamped", "swiglu", "swiglu_backward", "transpose_experts", "combine_backward",
        "route_backward", "permute_backward", "grouped_wgrad", "MoETrainingLayer", "router_prepare",
        "router_topk", "tile_rows", "untile_rows", "tile_weights", "TiledWeights", "even_rows",
        "grouped_glu_gemm_tiled", "grouped_glu_gemm_gather_tiled", "grouped_down_gemm_tiled",
        "tile_fp8_weights", "untile_fp8_rows", "grouped_gemm_tiled", "swiglu_tiled", "swiglu_backward_tiled",
        "grouped_wgrad_tiled", "training_weights")


def __getattr__(name):
    # the binding imports torch; load it on first use so that the input
    # generators and accounting stay importable without it
    if name in _API:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
