"""CPU oracle for the routed NVFP4 mixture-of-experts FFN (test infrastructure).

This package is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and shares no code, table or helper with
it.  It is plain and slow on purpose: fp64 NumPy, per-route loops, one
library matmul per projection, no blocking or fusion.

What it computes (one routed-MoE step of a decode/verify batch):
  router_logits   the router projection that produces the routing logits
  route_topk      softmax top-k routing with renormalised gate weights
  bucket_routes   per-expert route counts, offsets, active list, stable order
  moe_output      per route: SiLU(W_gate x) * (W_up x), then W_down; weighted
                  sum over each token's k routes in slot order
  shared_expert_output  the dense BF16 shared expert for every token

Sources: the routing rule of the fused MoE routing kernel (page "How I forked
vLLM and made Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section
"5. Hand-written kernels", paragraph "Fused MoE routing"); the routed chain of
the SM70 design note (page "Persistent execution for Flash-Next GGUF on SM70",
sections "What the measurements establish", "First implementation boundary"
and "Router: selection and expert-task production").

Every function here has pins in tests/ (closed forms, brute force, library
reductions, invariants); none is "parity unpinned".
"""

from .formats import (
    E2M1_VALUES,
    e4m3_table,
    bf16_bits_to_f64,
    unpack_nibbles,
    dequant_nvfp4,
)
from .route import route_topk, selection_order, renormalised_weights
from .router import router_logits
from .buckets import bucket_routes
from .ffn import expert_route_output, moe_output, ExpertDecoder
from .shared import shared_expert_output

__all__ = [
    "shared_expert_output",
    "E2M1_VALUES",
    "e4m3_table",
    "bf16_bits_to_f64",
    "unpack_nibbles",
    "dequant_nvfp4",
    "router_logits",
    "route_topk",
    "selection_order",
    "renormalised_weights",
    "bucket_routes",
    "expert_route_output",
    "moe_output",
    "ExpertDecoder",
]
