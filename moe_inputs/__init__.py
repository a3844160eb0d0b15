"""Seeded synthetic inputs for the routed NVFP4 mixture-of-experts FFN.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random tensors, encodes expert weights to NVFP4 and forms
router logits; it implements none of the routed-MoE step itself (no top-k, no
bucketing, no dequantisation, no expert FFN, no combine).

Workload shapes and distributions follow the five configurations the routed
MoE step is measured on: a tiny case (T=4, H=256, I=128, E=8, top-2) and four
cases at H=2048, I=512, E=512, top-10 with T = 4, 32, 256 and 4096 tokens;
the Flash-Next expert shape (H=2560, I=640) is an extra configuration.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .nvfp4_encode import encode_nvfp4, encode_e4m3, encode_e2m1
from .generate import (
    Workload,
    make_workload,
    make_expert_bank,
    f64_to_bf16_bits,
    router_logits,
)

__all__ = [
    "CONFIGS",
    "WorkloadConfig",
    "get_config",
    "encode_nvfp4",
    "encode_e4m3",
    "encode_e2m1",
    "Workload",
    "make_workload",
    "make_expert_bank",
    "f64_to_bf16_bits",
    "router_logits",
]
