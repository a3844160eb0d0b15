"""Router projection (test infrastructure): the routing logits from the tokens.

logits[t, e] = fl32( sum_h x[t, h] * W_r[e, h] ): every bf16 activation and
fp32 router weight is exact in fp64, so is each product, and the sum is taken
in fp64 and rounded once to fp32.  The router is a projection followed by the
selection (page "Persistent execution for Flash-Next GGUF on SM70", section
"Router: selection and expert-task production"); the projection's precision
is not stated on the pages, and this is the plain reading of it (one rounding,
at the end).  One library matmul, no blocking.
"""

import numpy as np

from .formats import bf16_bits_to_f64


def router_logits(x_bf16: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """x_bf16: [T, H] bf16 bit patterns (uint16); w_router: [E, H] float32 ->
    logits [T, E] float32."""
    x = bf16_bits_to_f64(np.asarray(x_bf16, np.uint16))
    w = np.asarray(w_router, np.float32).astype(np.float64)
    return (x @ w.T).astype(np.float32)
