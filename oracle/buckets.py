"""Route bucketing: group the T*k routes by expert (test infrastructure).

The fused routing kernel follows top-k with counts, a scan, expert ids and a
scatter (page "How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x
faster on one GPU", section "5. Hand-written kernels", paragraph "Fused MoE
routing").  The SM70 design note asks for a compact expert-presence list and
the original route positions, preserving route order, without sorting or
gathering token features (page "Persistent execution for Flash-Next GGUF on
SM70", section "First implementation boundary", step 1).

Reading: routes are identified by their flat id r = t*k + j; the bucket order
is stable, i.e. routes sorted by (expert, r); no padding in the exported
layout.
"""

from __future__ import annotations

import numpy as np


def bucket_routes(topk_idx: np.ndarray, E: int) -> dict:
    """Returns expert_count [E], expert_offset [E+1], active_experts [E]
    (ascending ids with a route, then -1), n_active, route_src [R] (flat route
    ids in bucket order) and route_pos [R] (inverse of route_src)."""
    flat = [int(e) for e in np.asarray(topk_idx).reshape(-1)]
    R = len(flat)
    count = np.zeros(E, dtype=np.int32)
    for e in flat:
        count[e] += 1
    offset = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offset[e + 1] = offset[e] + count[e]
    active_list = [e for e in range(E) if count[e] > 0]
    active = np.full(E, -1, dtype=np.int32)
    active[: len(active_list)] = active_list
    route_src = np.array(sorted(range(R), key=lambda r: (flat[r], r)), dtype=np.int32)
    route_pos = np.zeros(R, dtype=np.int32)
    for p, r in enumerate(route_src):
        route_pos[r] = p
    return {
        "expert_count": count,
        "expert_offset": offset,
        "active_experts": active,
        "n_active": np.int32(len(active_list)),
        "route_src": route_src,
        "route_pos": route_pos,
    }
