"""The expert kernels' work lists on the GPU, through the C ABI.

Above 16 tokens the row-dot kernels take their experts from a list sorted by
route count, and on the MFMA path every expert contributes one work item per
chunk of up to 128 routes.  moe_step builds both lists at the end of its
bucketing kernel; moe_expert_ffn builds them in a kernel of its own.  Both
must give the same output bit for bit (the lists only decide which workgroup
computes what), and the edges of the chunking (an expert with exactly 128 or
129 routes, E above 512 and not a multiple of 8, the smallest batch that
sorts the row-dot experts) must match the oracle.
"""

import numpy as np
import pytest
import torch

import sparse_moe_expert_amd as sme
from gpu_harness import (
    DEV,
    assert_buckets,
    assert_output,
    assert_route,
    collect,
    device_packed,
    device_weights,
    oracle_all,
    to_dev,
    x_bits,
)
from moe_inputs import make_workload

pytestmark = pytest.mark.gpu


def _run(wl, logits, bias, path):
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path=path)
    st.run(x_bits(wl.x), to_dev(logits.astype(np.float32)),
           None if bias is None else to_dev(bias.astype(np.float32)), device_weights(wl.bank),
           packed=device_packed(wl.bank) if path == "packed" else None)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("name", ["verify_t32", "decode_t256_zipf", "prefill_t4096"])
def test_step_lists_equal_ffn_lists(name):
    """moe_step (lists from the bucketing kernel) and moe_route_bucket +
    moe_expert_ffn (lists from the FFN's own kernel) give the same output."""
    wl = make_workload(name)
    a = _run(wl, wl.logits, wl.bias, "step")
    b = _run(wl, wl.logits, wl.bias, "calls")
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))


def _forced(T, H, I, E, k, experts, seed):
    """A workload whose every token picks the given k experts."""
    from dataclasses import replace
    from moe_inputs.configs import get_config
    cfg = replace(get_config("tiny"), name="work_list_edge", H=H, I=I, E=E, k=k, T=T)
    wl = make_workload(cfg, x_seed=seed)
    bias = np.zeros(E, np.float32)
    bias[list(experts)] = 50.0
    return wl, bias


@pytest.mark.parametrize("path", ["step", "packed", "calls"])
@pytest.mark.parametrize("T", [128, 129])
def test_chunk_boundary(T, path):
    """Every token on the same 4 of 40 experts: T routes per expert, exactly
    one full 128-route chunk (T = 128) or one full chunk and one route
    (T = 129), on the MFMA path."""
    chosen = [3, 17, 18, 39]
    wl, bias = _forced(T, 256, 128, 40, 4, chosen, seed=T)
    st = _run(wl, wl.logits, bias, path)
    g = collect(st)
    idx, w, b, y = oracle_all(wl.x, wl.logits, bias, wl.bank, wl.k)
    assert sorted(np.unique(idx)) == chosen and np.all(b["expert_count"][chosen] == T)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    err, rms = assert_output(g["y"], y, f"chunk boundary T={T}")
    print(f"[chunk boundary] T={T} path={path}: every token, max_err={err:.3e} rms={rms:.3e}", flush=True)


@pytest.mark.parametrize("path", ["step", "packed", "calls"])
@pytest.mark.parametrize("T", [17, 70])
def test_wide_expert_count(T, path):
    """E = 1000 (above 512, not a multiple of 8), k = 8: T = 17 is the
    smallest batch whose row-dot experts come sorted; T = 70 takes the MFMA
    path (on the standard layout only the experts with 16 or more routes)."""
    from dataclasses import replace
    from moe_inputs.configs import get_config
    cfg = replace(get_config("tiny"), name="work_list_wide", H=256, I=128, E=1000, k=8, T=T)
    wl = make_workload(cfg, x_seed=5)
    # a skewed bias: a few experts take many routes
    bias = np.zeros(1000, np.float32)
    bias[[1, 500, 999]] = [3.0, 2.5, 2.0]
    st = _run(wl, wl.logits, bias, path)
    g = collect(st)
    idx, w, b, y = oracle_all(wl.x, wl.logits, bias, wl.bank, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, f"E=1000 T={T}")


@pytest.mark.parametrize("path", ["step", "packed", "calls"])
@pytest.mark.parametrize("T,E,k", [(17, 1, 1), (200, 1, 1), (70, 8, 8)])
def test_every_token_on_every_expert(T, E, k, path):
    """k = E: every expert takes every token.  E = 1 at T = 17 (one row-dot
    expert in the sorted list) and T = 200 (one expert, a full 128-route
    chunk and a 72-route one on the MFMA path); E = k = 8 at T = 70 (eight
    MFMA items of 70 routes)."""
    from dataclasses import replace
    from moe_inputs.configs import get_config
    cfg = replace(get_config("tiny"), name="work_list_all", H=256, I=128, E=E, k=k, T=T)
    wl = make_workload(cfg, x_seed=9)
    st = _run(wl, wl.logits, None, path)
    g = collect(st)
    idx, w, b, y = oracle_all(wl.x, wl.logits, None, wl.bank, wl.k)
    assert np.all(b["expert_count"] == T)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, f"k=E={E} T={T}")
