"""MI355X-native flow-matching action-expert decision.

The compute lives in ``libphx_expert.so`` (hand-written gfx950 HIP kernels
behind the C ABI of ``include/phx_expert.h``); ``binding`` exposes the same
calls through ctypes and ``expert`` wraps them around torch device tensors.
"""
from .binding import (PHX_BLOCK_DECODER, PHX_BLOCK_DIT, PHX_DTYPE_BF16, PHX_DTYPE_F32, PHX_MASK_FULL, PHX_FLAG_MULTI_KERNEL, PHX_FLAG_NO_GRAPH, PHX_FLAG_TIMELINE,
                      PHX_FLAG_PAIRED_ACT, PHX_FLAG_BF16_ACT, PHX_FLAG_WEIGHTS_INT8,
                      PhxError, load_library, make_config, phx_expert_create, phx_expert_decide, phx_expert_destroy,
                      phx_expert_kernels_per_decision, phx_expert_launch_node, phx_expert_load_prefix_kv,
                      phx_expert_node_info, phx_expert_status, phx_expert_timeline, phx_expert_validate_config,
                      phx_expert_weights_bytes, phx_last_error)

__all__ = ["PHX_BLOCK_DECODER", "PHX_BLOCK_DIT", "PHX_DTYPE_BF16", "PHX_DTYPE_F32", "PHX_MASK_FULL", "PHX_FLAG_MULTI_KERNEL", "PHX_FLAG_NO_GRAPH", "PHX_FLAG_TIMELINE",
           "PHX_FLAG_PAIRED_ACT", "PHX_FLAG_BF16_ACT", "PHX_FLAG_WEIGHTS_INT8",
           "PhxError", "load_library", "make_config", "phx_expert_create", "phx_expert_decide", "phx_expert_destroy",
           "phx_expert_kernels_per_decision", "phx_expert_launch_node", "phx_expert_load_prefix_kv",
           "phx_expert_node_info", "phx_expert_status", "phx_expert_timeline", "phx_expert_validate_config",
           "phx_expert_weights_bytes", "phx_last_error"]
