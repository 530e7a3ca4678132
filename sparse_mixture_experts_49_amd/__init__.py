"""MI355X-native (gfx950) forward pass of the sparsely-gated Mixture-of-Experts layer.

The layer runs in hand-written HIP kernels behind the C ABI of
libmoe_mi355x.so (header: include/moe_mi355x.h); this package is its ctypes
binding.  Build the library with ``python -m sparse_mixture_experts_49_amd.build``.
"""
from .binding import (ENTRY_POINTS, MOE_CAPACITY_DROP, MOE_CAPACITY_REROUTE, MOE_FFN_AUTO, MOE_FFN_STREAM, MOE_FFN_TILED, MOE_H_AUTO,
                      MOE_H_BF16, MOE_H_SPLIT, Desc, MoeError, Routing, Weights, alloc_h,
                      alloc_workspace, forward, load_library, moe_combine, moe_ffn_down,
                      moe_ffn_up, moe_ffn_up_gather, moe_forward, moe_forward_noalloc, moe_read_probe, moe_grouped_ffn, moe_permute, moe_query_plan,
                      moe_route, moe_shared_ffn, moe_workspace_size)

__all__ = ["ENTRY_POINTS", "MOE_CAPACITY_DROP", "MOE_CAPACITY_REROUTE", "MOE_FFN_AUTO", "MOE_FFN_STREAM", "MOE_FFN_TILED", "MOE_H_AUTO",
           "MOE_H_BF16", "MOE_H_SPLIT", "Desc", "MoeError", "Routing", "Weights", "alloc_h",
           "alloc_workspace", "forward", "load_library", "moe_combine", "moe_ffn_down",
           "moe_ffn_up", "moe_ffn_up_gather", "moe_forward", "moe_forward_noalloc", "moe_read_probe", "moe_grouped_ffn", "moe_permute", "moe_query_plan",
           "moe_route", "moe_shared_ffn", "moe_workspace_size"]
