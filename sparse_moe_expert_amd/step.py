"""One routed-MoE step with preallocated outputs, for graph capture and reuse.

MoeStep owns every output and the workspace for fixed sizes (T, H, I, E, k)
and enqueues the three library calls on torch's current stream.  Because no
call allocates or synchronises, `run` can be captured in a torch.cuda.CUDAGraph
(a HIP graph under ROCm) and replayed after the input tensors' contents change.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from ._lib import (
    ExpertWeights,
    empty_buckets,
    make_workspace,
    moe_bucket_routes,
    moe_expert_ffn,
    moe_route_bucket,
    moe_route_topk,
)


def expert_weights_from_numpy(bank, device) -> ExpertWeights:
    """Copy an NVFP4 expert bank (numpy arrays w_gate, s_gate, ..., g_scale) to the device."""
    dev = torch.device(device)
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)  # noqa: E731
    return ExpertWeights(
        to(bank.w_gate, torch.uint8), to(bank.s_gate, torch.uint8),
        to(bank.w_up, torch.uint8), to(bank.s_up, torch.uint8),
        to(bank.w_down, torch.uint8), to(bank.s_down, torch.uint8),
        to(bank.g_scale, torch.float32))


class MoeStep:
    """fused_routing: route and bucket with moe_route_bucket (one call) instead
    of moe_route_topk followed by moe_bucket_routes; the outputs are identical."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device, fused_routing: bool = True):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.fused_routing = fused_routing
        self.device = torch.device(device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=self.device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=self.device)
        self.buckets = empty_buckets(T, E, k, self.device)
        self.workspace = make_workspace(T, H, I, E, k, self.device)
        self.y = torch.empty((T, H), dtype=torch.bfloat16, device=self.device)

    def route(self, logits: torch.Tensor, bias: Optional[torch.Tensor]):
        moe_route_topk(logits, bias, self.k, self.topk_idx, self.topk_w)

    def bucket(self):
        moe_bucket_routes(self.topk_idx, self.E, self.buckets)

    def route_bucket(self, logits: torch.Tensor, bias: Optional[torch.Tensor]):
        moe_route_bucket(logits, bias, self.k, self.topk_idx, self.topk_w, self.buckets)

    def ffn(self, x: torch.Tensor, weights: ExpertWeights, stage: int = 3):
        moe_expert_ffn(x, weights, self.topk_w, self.buckets, self.workspace, self.y, stage=stage)

    def routing(self, logits: torch.Tensor, bias: Optional[torch.Tensor]):
        if self.fused_routing:
            self.route_bucket(logits, bias)
        else:
            self.route(logits, bias)
            self.bucket()

    def run(self, x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor],
            weights: ExpertWeights) -> torch.Tensor:
        self.routing(logits, bias)
        self.ffn(x, weights)
        return self.y
