"""Softmax top-k routing with renormalised gate weights (test infrastructure).

Follows the fused MoE routing kernel's contract: per token a softmax over the
experts, top-k by arg-max on the scores with the lowest expert id winning
ties (page "How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x faster
on one GPU", section "5. Hand-written kernels", paragraph "Fused MoE
routing"), and the router contract of the SM70 note: keep the softmax, the tie
rule, the normalisation and the route order; ties resolve to the lowest expert
index (page "Persistent execution for Flash-Next GGUF on SM70", section
"Router: selection and expert-task production").

Readings where the pages are brief:
  * z = fl32(logit + bias): the optional per-expert bias is added to the
    logits once, in fp32, and feeds both the selection and the softmax.
  * Selection compares the fp32 z values (softmax is strictly increasing, so
    the set equals the top-k of the probabilities in exact arithmetic);
    -0.0 and +0.0 compare equal.
  * Slot j of a token holds its j-th choice: z descending, id ascending.
  * Weights: softmax over all E experts in fp64, then divided by the sum over
    the selected k (renormalised to sum 1); no epsilon, no extra scaling.
"""

from __future__ import annotations

import numpy as np


def _selection_key(value: float, expert: int):
    # larger score first; among equal scores the lower expert id first
    return (-value, expert)


def selection_order(z_row, k: int) -> list:
    """The k experts a token selects, in slot order (plain sort of all experts)."""
    keyed = sorted((_selection_key(float(v), e) for e, v in enumerate(z_row)))
    return [e for _, e in keyed[:k]]


def _renormalise(p_selected: np.ndarray) -> np.ndarray:
    return p_selected / p_selected.sum()


def renormalised_weights(z_row, selected) -> np.ndarray:
    """Softmax over all experts in fp64, restricted to `selected` and renormalised."""
    z = np.asarray(z_row, dtype=np.float64)
    ex = np.exp(z - z.max())
    p = ex / ex.sum()
    return _renormalise(p[np.asarray(selected, dtype=np.int64)])


def biased_scores(logits: np.ndarray, bias) -> np.ndarray:
    """z = fl32(logits + bias): one IEEE fp32 addition per element."""
    z = np.asarray(logits, dtype=np.float32)
    if bias is None:
        return z.copy()
    return (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def route_topk(logits: np.ndarray, bias, k: int):
    """Returns (topk_idx int32 [T, k], topk_w float64 [T, k])."""
    z = biased_scores(logits, bias)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        sel = selection_order(z[t], k)
        idx[t] = sel
        w[t] = renormalised_weights(z[t], sel)
    return idx, w
