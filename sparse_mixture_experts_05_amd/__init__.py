"""MI355X (gfx950) top-k MoE SwiGLU layer: forward, training backward, the
shared-neuron residual layer and an allocation-free forward.

The compute path is libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h); this package is its thin Python binding. PyTorch supplies
device memory and streams only.
"""
from .abi import (MOE_BF16, MOE_F32, MOE_SOFTMAX_THEN_TOPK, MOE_TOPK_THEN_SOFTMAX, MoEConfig, MoEError,
                  load_library, moe_backward, moe_capacity, moe_check, moe_combine, moe_debug_build,
                  moe_debug_word_offset, moe_forward, moe_forward_noalloc, moe_forward_residual, moe_forward_train,
                  moe_grouped_swiglu, moe_noalloc_scratch_bytes, moe_permute, moe_profile_read, moe_profile_select,
                  moe_residual_workspace_bytes, moe_route, moe_train_workspace_bytes, moe_workspace_bytes,
                  use_library, workspace)
from .layer import MoEFunction, MoELayer

__all__ = ["MoEConfig", "MoEError", "MoEFunction", "MoELayer", "load_library", "use_library", "moe_backward",
           "moe_capacity", "moe_check", "moe_combine", "moe_debug_build", "moe_debug_word_offset", "moe_forward",
           "moe_forward_noalloc", "moe_forward_residual", "moe_forward_train", "moe_grouped_swiglu",
           "moe_noalloc_scratch_bytes", "moe_permute", "moe_profile_read", "moe_profile_select",
           "moe_residual_workspace_bytes", "moe_route", "moe_train_workspace_bytes", "moe_workspace_bytes",
           "workspace", "MOE_BF16", "MOE_F32", "MOE_TOPK_THEN_SOFTMAX", "MOE_SOFTMAX_THEN_TOPK"]
