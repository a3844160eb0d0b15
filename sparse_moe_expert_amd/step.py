"""One routed-MoE step with preallocated outputs, for graph capture and reuse.

MoeStep owns every output and the workspace for fixed sizes (T, H, I, E, k)
and enqueues the library calls on torch's current stream.  Because no
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
    moe_step,
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
    """Outputs and workspace for one step of fixed sizes, and the ways to run it.

    path "step": moe_step (the whole step in one call).  "packed":
    moe_step_packed, with the weights' packed copy passed to run().  "calls":
    moe_route_bucket then moe_expert_ffn.  "calls_unfused": moe_route_topk,
    moe_bucket_routes, moe_expert_ffn.  All of them produce the same outputs."""

    PATHS = ("step", "packed", "calls", "calls_unfused")

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device, path: str = "step"):
        if path not in self.PATHS:
            raise ValueError(f"path must be one of {self.PATHS}")
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.path = path
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

    def routing(self, logits: torch.Tensor, bias: Optional[torch.Tensor]):
        if self.path == "calls_unfused":
            self.route(logits, bias)
            self.bucket()
        else:
            self.route_bucket(logits, bias)

    def ffn(self, x: torch.Tensor, weights: ExpertWeights, stage: int = 3):
        moe_expert_ffn(x, weights, self.topk_w, self.buckets, self.workspace, self.y, stage=stage)

    def run(self, x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor],
            weights: ExpertWeights, packed: Optional[torch.Tensor] = None, stage: int = 3) -> torch.Tensor:
        """The step; stage 1 or 2 (paths "step" and "packed") runs one part of it."""
        if self.path in ("step", "packed"):
            if self.path == "packed" and packed is None:
                raise ValueError('path "packed" needs the packed weights (pack_weights)')
            moe_step(x, logits, bias, weights, self.k, self.topk_idx, self.topk_w, self.buckets,
                     self.workspace, self.y, packed=packed if self.path == "packed" else None, stage=stage)
        else:
            if stage != 3:
                raise ValueError('stages are run on paths "step" and "packed"')
            self.routing(logits, bias)
            self.ffn(x, weights)
        return self.y
