"""Routed mixture-of-experts forward for AMD MI355X (gfx950).

The compute path is libmoe.so (hand-written HIP kernels behind a C ABI,
include/moe.h); this package is its thin ctypes binding plus the seeded
synthetic input generator.
"""
from ._lib import (EXPORTS, LIB_PATH, MOE_NUM_STAGES, MOE_WEIGHT_DTYPE,  # noqa: F401
                   MOE_WEIGHT_FP8_E4M3, MOE_WEIGHT_MXFP4, STAGES, ExpertWeights, MoeError, Placement,
                   RouteConfig, load, moe_combine, moe_experts, moe_experts_ex, moe_forward,
                   moe_forward_ex, moe_forward_noalloc, moe_forward_workspace,
                   moe_load_accumulate, moe_log2phy, moe_permute, moe_route)
