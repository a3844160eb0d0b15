"""The small-batch step: moe_step up to 40 routes selects inside its gate/up
launch (one workgroup per route and row tile) and buckets beside it, then
runs its route-slot down/unroute; rows of one 16-byte chunk per lane at H =
2048, of several chunks per lane at other sizes (H = 2560 of the Flash-Next
expert), and likewise for the down rows.

Every output (ids, weights, the six bucket arrays, y) must equal bit for bit
what moe_route_bucket + moe_expert_ffn produce on the same inputs, and match
the oracle; shapes cover one to four tokens, k = 1, k = 32, E = 64 and
E = 1000 (past the small step's 512 experts: the general path, which must
give the same outputs), a bias, ties, both weight paths, guard regions around y and the
workspace, and graph replays with changed inputs.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import sparse_moe_expert_amd as sme
from gpu_harness import (DEV, assert_buckets, assert_output, assert_route, collect, device_packed, device_weights,
                         oracle_all, to_dev, x_bits)
from moe_inputs import make_workload
from moe_inputs.configs import get_config

pytestmark = pytest.mark.gpu


def _wl(T, E, k, seed, I=512, H=2048):
    cfg = replace(get_config("decode_t4"), name="small_step", T=T, E=E, k=k, I=I, H=H)
    return make_workload(cfg, x_seed=seed)


# (T, E, k, I, bias, ties): all at H = 2048 and at most 40 routes
CASES = [(4, 512, 10, 512, False, False), (1, 512, 10, 512, True, False), (2, 512, 10, 512, False, True),
         (3, 512, 10, 512, True, False), (4, 512, 1, 512, False, False), (1, 512, 32, 512, False, False),
         (4, 64, 10, 512, True, False), (5, 1000, 8, 512, False, False), (4, 256, 10, 256, False, False),
         (2, 512, 10, 1024, False, False)]


@pytest.mark.parametrize("path", ["step", "packed"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_E%d_k%d_I%d_bias%d_ties%d" % c)
def test_small_step_equals_calls_and_oracle(case, path):
    _check_small_step(*case, path=path)


# (T, E, k, H, I, bias, ties): rows of several chunks per lane - the
# Flash-Next expert (H = 2560, I = 640: 80 and 20 chunks), H = 1280 and 3072
# (40 and 96 chunks), and H = 2048 with I = 4096 (one-chunk gate/up rows,
# 128-chunk down rows); each within the route-slot down's register bound
NC_CASES = [(4, 512, 10, 2560, 640, False, False), (2, 512, 10, 2560, 640, True, True),
            (4, 64, 10, 1280, 768, False, False), (4, 16, 4, 3072, 640, True, False),
            (1, 16, 4, 2048, 4096, False, False)]


@pytest.mark.parametrize("path", ["step", "packed"])
@pytest.mark.parametrize("case", NC_CASES, ids=lambda c: "T%d_E%d_k%d_H%d_I%d_bias%d_ties%d" % c)
def test_small_step_several_chunks_equals_calls_and_oracle(case, path):
    T, E, k, H, I, with_bias, ties = case
    _check_small_step(T, E, k, I, with_bias, ties, path=path, H=H)


def _check_small_step(T, E, k, I, with_bias, ties, path, H=2048):
    print(f"[small step] T={T} E={E} k={k} H={H} I={I} bias={with_bias} ties={ties} path={path}", flush=True)
    wl = _wl(T, E, k, 60 + T + k, I=I, H=H)
    logits = wl.logits
    if ties:
        logits = (np.round(logits * 4.0) / 4.0).astype(np.float32)
    bias = (0.5 * np.random.default_rng(T).standard_normal(E)).astype(np.float32) if with_bias else None
    W = device_weights(wl.bank)
    a = sme.MoeStep(T, wl.H, I, E, k, DEV, path=path)
    a.run(x_bits(wl.x), to_dev(logits), None if bias is None else to_dev(bias), W,
          packed=device_packed(wl.bank) if path == "packed" else None)
    b = sme.MoeStep(T, wl.H, I, E, k, DEV, path="calls")
    b.run(x_bits(wl.x), to_dev(logits), None if bias is None else to_dev(bias), W)
    torch.cuda.synchronize()
    assert torch.equal(a.topk_idx, b.topk_idx)
    assert torch.equal(a.topk_w.view(torch.int32), b.topk_w.view(torch.int32))
    for ta, tb in zip(a.buckets, b.buckets):
        assert torch.equal(ta, tb)
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))
    g = collect(a)
    idx, w, bk, y = oracle_all(wl.x, logits, bias, wl.bank, k)
    assert_route(g, idx, w)
    assert_buckets(g, bk)
    assert_output(g["y"], y, f"small step T={T} E={E} k={k} H={H} I={I}")


def test_small_step_guard_regions():
    wl = make_workload("decode_t4", x_seed=19)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    step = sme.MoeStep(T, H, I, E, k, DEV, path="step")
    ws_bytes = sme.moe_step_workspace_size(T, H, I, E, k)
    big_ws = torch.zeros(ws_bytes + 512, dtype=torch.uint8, device=DEV)
    big_ws[:256] = 0xA5
    big_ws[256 + ws_bytes:] = 0x5A
    step.workspace = big_ws[256: 256 + ws_bytes]
    big_y = torch.full((T + 2, H), 3.0, dtype=torch.bfloat16, device=DEV)
    step.y = big_y[1: T + 1]
    step.run(x_bits(wl.x), to_dev(wl.logits), None, device_weights(wl.bank))
    torch.cuda.synchronize()
    assert torch.all(big_ws[:256] == 0xA5) and torch.all(big_ws[256 + ws_bytes:] == 0x5A)
    assert torch.all(big_y[0] == 3.0) and torch.all(big_y[T + 1] == 3.0)
    idx, w, b, y = oracle_all(wl.x, wl.logits, None, wl.bank, k)
    assert_output(big_y[1: T + 1].float().cpu().numpy().astype(np.float64), y, "guarded small step")


@pytest.mark.parametrize("name,path", [("decode_t4", "step"), ("decode_t4", "packed"), ("flashnext_t4", "step"),
                                       ("verify_t32", "step"), ("decode_t256_zipf", "packed")])
def test_step_stages_compose(name, path):
    """moe_step_stage 1 then 2 gives moe_step's outputs bit for bit (the small
    step's two launches at decode_t4 and, with rows of several chunks per
    lane, at the Flash-Next shape; routing, buckets and gate/up, then down
    and the unroute, at the larger batches)."""
    wl = make_workload(name, x_seed=77)
    W = device_weights(wl.bank)
    pk = device_packed(wl.bank) if path == "packed" else None
    bias = None if wl.bias is None else to_dev(wl.bias)
    full = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path=path)
    full.run(x_bits(wl.x), to_dev(wl.logits), bias, W, packed=pk)
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path=path)
    st.run(x_bits(wl.x), to_dev(wl.logits), bias, W, packed=pk, stage=1)
    st.run(x_bits(wl.x), to_dev(wl.logits), bias, W, packed=pk, stage=2)
    torch.cuda.synchronize()
    assert torch.equal(full.topk_idx, st.topk_idx)
    assert torch.equal(full.topk_w.view(torch.int32), st.topk_w.view(torch.int32))
    for ta, tb in zip(full.buckets, st.buckets):
        assert torch.equal(ta, tb)
    assert torch.equal(full.y.view(torch.int16), st.y.view(torch.int16))
