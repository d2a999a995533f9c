"""MI355X (gfx950) top-k MoE SwiGLU layer, forward pass.

The compute path is libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h); this package is its thin Python binding. PyTorch supplies
device memory and streams only.
"""
from .abi import (MOE_BF16, MOE_F32, MOE_SOFTMAX_THEN_TOPK, MOE_TOPK_THEN_SOFTMAX, MoEConfig, MoEError,
                  load_library, moe_capacity, moe_check, moe_combine, moe_forward, moe_grouped_swiglu,
                  moe_permute, moe_profile_read, moe_profile_select, moe_route, moe_workspace_bytes, workspace)
from .layer import MoELayer

__all__ = ["MoEConfig", "MoEError", "MoELayer", "load_library", "moe_capacity", "moe_check", "moe_combine",
           "moe_forward", "moe_grouped_swiglu", "moe_permute", "moe_route", "moe_workspace_bytes",
           "moe_profile_read", "moe_profile_select", "workspace", "MOE_BF16", "MOE_F32",
           "MOE_TOPK_THEN_SOFTMAX", "MOE_SOFTMAX_THEN_TOPK"]
