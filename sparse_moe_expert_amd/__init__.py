"""Routed NVFP4 mixture-of-experts FFN on MI355X (gfx950).

A C-ABI HIP library (include/moe.h) with three calls per routed-MoE step:
moe_route_topk -> moe_bucket_routes -> moe_expert_ffn (or the whole step in
one call, moe_step), bound here for torch tensors.  PyTorch provides device memory and the stream; the kernels are the
library's own.
"""

from ._lib import (
    Buckets,
    ExpertWeights,
    LIB_PATH,
    MoeError,
    SIGNATURES,
    empty_buckets,
    load_library,
    make_workspace,
    moe_bucket_routes,
    moe_expert_ffn,
    moe_expert_ffn_per_route,
    moe_expert_ffn_workspace_size,
    moe_route_bucket,
    moe_router_logits,
    moe_router_route_bucket,
    moe_route_topk,
    moe_shared_expert,
    moe_step_shared,
    moe_status_string,
    moe_packed_weights_size,
    moe_step,
    moe_step_noalloc,
    moe_step_workspace_size,
    NOALLOC_SCRATCH_BYTES,
    pack_weights,
)
from .step import MoeStep, expert_weights_from_numpy

__all__ = [
    "Buckets",
    "ExpertWeights",
    "LIB_PATH",
    "MoeError",
    "SIGNATURES",
    "empty_buckets",
    "load_library",
    "make_workspace",
    "moe_bucket_routes",
    "moe_expert_ffn",
    "moe_expert_ffn_per_route",
    "moe_expert_ffn_workspace_size",
    "moe_route_bucket",
    "moe_router_logits",
    "moe_router_route_bucket",
    "moe_route_topk",
    "moe_shared_expert",
    "moe_step_shared",
    "moe_status_string",
    "moe_packed_weights_size",
    "moe_step",
    "moe_step_noalloc",
    "moe_step_workspace_size",
    "NOALLOC_SCRATCH_BYTES",
    "pack_weights",
    "MoeStep",
    "expert_weights_from_numpy",
]
