"""Routed expert FFN and weighted unroute in fp64 (test infrastructure).

The expert path is gate/up -> SiLU * multiply -> down, followed by a weighted
unroute (page "Persistent execution for Flash-Next GGUF on SM70", section
"What the measurements establish": gate/up fused with SiLU/multiply, down fused
with weighted unroute; section "First implementation boundary", flowchart and
step 4: routes are summed in a fixed order).

Per route (t, j) with expert e = topk_idx[t, j]:
    x  = bf16 token t, exactly in fp64
    g  = W_gate[e] x,   u = W_up[e] x
    a  = SiLU(g) * u,   SiLU(v) = v / (1 + exp(-v))
    o  = W_down[e] a
and y[t] = sum_{j=0}^{k-1} topk_w[t, j] * o_(t, j), in slot order j = 0..k-1.

Everything is fp64; the only rounding is fp64's own.  Weights are the exact
NVFP4 values (see formats.dequant_nvfp4).  No expert batching: one matvec per
projection per route.
"""

from __future__ import annotations

from collections import OrderedDict

import numpy as np

from .formats import bf16_bits_to_f64, dequant_nvfp4


def silu(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


class ExpertDecoder:
    """Dequantised fp64 matrices of one expert bank, decoded on first use.

    `bank` is any object with attributes w_gate, s_gate, w_up, s_up, w_down,
    s_down (uint8 arrays [E, rows, ...]) and g_scale (float32 [E, 3]).
    Decoded experts are memoised (most recent `cache` experts) only to avoid
    decoding the same bytes twice; the values are those of dequant_nvfp4.
    """

    def __init__(self, bank, cache: int = 16):
        self.bank = bank
        self.cache = cache
        self._memo: "OrderedDict[int, tuple]" = OrderedDict()

    def matrices(self, e: int):
        if e in self._memo:
            self._memo.move_to_end(e)
            return self._memo[e]
        b = self.bank
        g = np.asarray(b.g_scale, dtype=np.float32)
        mats = (
            dequant_nvfp4(b.w_gate[e], b.s_gate[e], float(g[e, 0])),
            dequant_nvfp4(b.w_up[e], b.s_up[e], float(g[e, 1])),
            dequant_nvfp4(b.w_down[e], b.s_down[e], float(g[e, 2])),
        )
        self._memo[e] = mats
        if len(self._memo) > self.cache:
            self._memo.popitem(last=False)
        return mats


def expert_route_output(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                        w_down: np.ndarray) -> np.ndarray:
    """o = W_down (SiLU(W_gate x) * (W_up x)) for one route, fp64."""
    g = w_gate @ x
    u = w_up @ x
    return w_down @ (silu(g) * u)


def moe_output(x_bf16: np.ndarray, bank, topk_idx: np.ndarray, topk_w: np.ndarray,
               tokens=None, decoder: ExpertDecoder = None) -> np.ndarray:
    """y [len(tokens), H] fp64 for the given tokens (default: all)."""
    x_bf16 = np.asarray(x_bf16)
    T = x_bf16.shape[0]
    tokens = range(T) if tokens is None else list(tokens)
    dec = decoder if decoder is not None else ExpertDecoder(bank)
    H = x_bf16.shape[1]
    k = topk_idx.shape[1]
    out = np.zeros((len(tokens), H), dtype=np.float64)
    for row, t in enumerate(tokens):
        x = bf16_bits_to_f64(x_bf16[t])
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            wg, wu, wd = dec.matrices(int(topk_idx[t, j]))
            acc = acc + float(topk_w[t, j]) * expert_route_output(x, wg, wu, wd)
        out[row] = acc
    return out
