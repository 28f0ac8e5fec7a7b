"""MXFP4 (and MXFP8) routed-expert MoE layer for AMD MI355X (gfx950).

The compute lives in libmoe_mxfp4.so (hand-written HIP kernels behind a C
ABI declared in include/moe_mxfp4.h); ``ops`` is its ctypes binding.
Build the library with ``python -m mxfp4_routed_expert_top_amd.build``.
"""
from . import ops  # noqa: F401
from .ops import (ACT_BF16, ACT_MXFP4, ACT_MXFP4_BLOCKED, W_MXFP4, W_MXFP8,  # noqa: F401
                  MoeError, align_sort, alloc_stages, combine, expert_down, expert_gate_up,
                  forward_stages, mxfp4_forward, mxfp4_forward_layers, mxfp4_forward_router,
                  mxfp4_quantize, mxfp4_quantize_blocked, mxfp8_expert_down,
                  mxfp8_expert_gate_up, mxfp8_forward, mxfp8_quantize, mxfp8_workspace_size,
                  quantize_weights, route_topk, route_topk_gemm, weights_to_native,
                  workspace_size)
