"""Dense shared expert in fp64 (test infrastructure).

Besides its routed experts, the Flash-Next MoE layer has a shared expert that
every token goes through.  Its weights stay BF16 when the rest is quantised
(page "How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x faster on one
GPU", section "2. FP8 for the dense layers": the shared experts are among the
layers kept in BF16), and its gate/up runs beside the routed work (page
"Persistent execution for Flash-Next GGUF on SM70", section "Opportunity sized
from the actual routes").  It is the same SwiGLU chain as a routed expert,
for every token and without a gate weight:

    y_t = W_down (SiLU(W_gate x_t) * (W_up x_t)),   SiLU(v) = v / (1 + exp(-v))

with x, W_gate [Is, H], W_up [Is, H] and W_down [H, Is] given as bf16 bit
patterns and evaluated exactly in fp64; the only rounding is fp64's own.
"""

from __future__ import annotations

import numpy as np

from .ffn import silu
from .formats import bf16_bits_to_f64


def shared_expert_output(x_bf16: np.ndarray, w_gate_bf16: np.ndarray, w_up_bf16: np.ndarray,
                         w_down_bf16: np.ndarray) -> np.ndarray:
    """[T, H] fp64 output of the shared expert for every token."""
    x = bf16_bits_to_f64(x_bf16)
    wg = bf16_bits_to_f64(w_gate_bf16)
    wu = bf16_bits_to_f64(w_up_bf16)
    wd = bf16_bits_to_f64(w_down_bf16)
    out = np.empty((x.shape[0], wd.shape[0]), dtype=np.float64)
    for t in range(x.shape[0]):               # one matvec per projection per token
        a = silu(wg @ x[t]) * (wu @ x[t])
        out[t] = wd @ a
    return out
