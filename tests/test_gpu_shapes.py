"""Row lengths whose 16-byte chunk count is not a power of two, on the GPU.

The Flash-Next expert as the pages size it (H = 2560, I = 640: 80 and 20
chunks per row) at the decode step (T = 4: the small step with multi-chunk
rows on the step paths, the multi-chunk gate/up and fused down/unroute
kernels on the separate calls) and at 256 tokens (the MFMA tiles with the packed copy;
on the standard layout the experts with fewer than 16 routes take the
multi-chunk gate/up, per-expert down and combine kernels), plus smaller
shapes that reach every chunk count the kernels are compiled for and rows
with a tail (chunks past the row read as zero).  Every output is compared
with the oracle (ids and buckets bit-exact, weights within 1e-6, y within
2e-2 * rms plus half a bf16 ulp).
"""

from dataclasses import replace

import numpy as np
import pytest

from gpu_harness import assert_buckets, assert_output, assert_route, oracle_all, run_gpu
from moe_inputs import make_workload
from moe_inputs.configs import get_config

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["step", "packed", "calls"])
@pytest.mark.parametrize("name", ["flashnext_t4", "flashnext_t256"])
def test_flash_next_expert_shape(name, path):
    wl = make_workload(name)
    print(f"[shape] {name} H={wl.H} I={wl.I} path={path}", flush=True)
    g = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    err, rms = assert_output(g["y"], y, name)
    print(f"[shape] {name} path={path}: every token, max_err={err:.3e} rms={rms:.3e} ratio={err / rms:.4f}",
          flush=True)


# (H, I, E, k, T): chunk counts per row (H/32, I/32) of 3 (one 16-lane pass
# with a tail), 5, 6, 12, 20, 24, 40, 80, 96 and 128.  Small batches take the
# fused down/unroute kernel when every route's h fits its LDS (64 KB) and the
# per-expert down tiles plus the combine otherwise (I = 2560 at T = 20, I =
# 4096 at T = 4); on the step paths those of at most 40 routes whose down
# fits take the small step (selection inside the gate/up launch, route-slot
# down/unroute); T = 70 takes the MFMA path as well.
ODD_ROW_SHAPES = [
    (96, 160, 8, 2, 4),
    (192, 384, 8, 3, 10),
    (640, 96, 16, 4, 20),
    (1280, 768, 32, 4, 10),
    (3072, 640, 16, 4, 4),
    (4096, 512, 16, 2, 4),
    (2048, 4096, 8, 2, 4),
    (2560, 640, 16, 4, 70),
    (384, 2560, 8, 2, 20),
]


@pytest.mark.parametrize("path", ["step", "packed", "calls"])
@pytest.mark.parametrize("shape", ODD_ROW_SHAPES, ids=lambda s: "H%d_I%d_E%d_k%d_T%d" % s)
def test_odd_row_lengths(shape, path):
    H, I, E, k, T = shape
    if path == "packed" and (H % 64 or I % 64):
        pytest.skip("packed weights need H and I multiples of 64")
    cfg = replace(get_config("tiny"), name="odd_rows", H=H, I=I, E=E, k=k, T=T)
    wl = make_workload(cfg, x_seed=31 + T)
    print(f"[odd rows] H={H} I={I} E={E} k={k} T={T} path={path}", flush=True)
    g = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, f"odd rows {shape}")
