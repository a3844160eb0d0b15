"""The synthetic workloads have the routing regimes their descriptions name.

Decode T=4 touches at most 40 distinct experts of ~1.77 MB; the biased T=32
batch reuses experts; the Zipf T=256 batch has hot experts with 30+ tokens and
many single-token experts; the T=4096 prefill chunk touches every expert with
about 80 tokens each.  Routing here is the oracle's.
"""

import numpy as np
import pytest

import oracle
from moe_inputs import CONFIGS, make_workload
from moe_inputs.configs import CONFIG_ORDER


def _counts(name):
    wl = make_workload(name, with_bank=False)
    idx, _ = oracle.route_topk(wl.logits, wl.bias, wl.k)
    return np.bincount(idx.reshape(-1), minlength=wl.E)


def test_shapes_and_determinism():
    a = make_workload("tiny")
    b = make_workload("tiny")
    assert a.x.shape == (4, 256) and a.logits.shape == (4, 8) and a.bias is None
    assert a.bank.w_gate.shape == (8, 128, 128) and a.bank.s_down.shape == (8, 256, 8)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.bank.w_down, b.bank.w_down)
    assert CONFIGS["decode_t4"].expert_bytes() == 1769472
    assert CONFIG_ORDER[1] == "decode_t4"


def test_decode_t4_unique_experts():
    c = _counts("decode_t4")
    assert 30 <= np.count_nonzero(c) <= 40 and c.sum() == 40


def test_verify_t32_reuse():
    c = _counts("verify_t32")
    assert c.max() >= 4 and 100 <= np.count_nonzero(c) <= 200


def test_zipf_t256_skew():
    c = _counts("decode_t256_zipf")
    nz = c[c > 0]
    assert c.max() >= 100 and (nz >= 30).sum() >= 10 and (nz == 1).sum() >= 10


def test_prefill_t4096_uniform():
    c = _counts("prefill_t4096")
    assert np.count_nonzero(c) == 512 and c.sum() == 40960 and c.max() < 160
