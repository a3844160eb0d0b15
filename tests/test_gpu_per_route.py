"""The no-reuse baseline (moe_expert_ffn_per_route) against the oracle.

Every route streams its own expert's weights; the result has the definition
of the reuse path.  Routing comes from moe_route_topk; the output is compared
on every token with the oracle (2e-2 * rms plus half a bf16 ulp), at the
workloads the reuse measurement covers (tiny, decode_t4, verify_t32), the
Flash-Next expert shape, edge shapes with tails and k = E, and bitwise
run-to-run determinism.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import DEV, assert_output, device_weights, shared_decoder, to_dev, x_bits
from moe_inputs import make_workload
from moe_inputs.configs import get_config

pytestmark = pytest.mark.gpu


def _per_route(wl, bias=None):
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    b = wl.bias if bias is None else bias
    sme.moe_route_topk(to_dev(wl.logits), None if b is None else to_dev(b.astype(np.float32)), k, idx, w)
    ws = sme.make_workspace(T, H, I, E, k, DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    sme.moe_expert_ffn_per_route(x_bits(wl.x), device_weights(wl.bank), idx, w, ws, y)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), y


@pytest.mark.parametrize("name", ["tiny", "decode_t4", "verify_t32", "flashnext_t4"])
def test_per_route_against_oracle(name):
    wl = make_workload(name)
    idx_g, w_g, y = _per_route(wl)
    idx, w = oracle.route_topk(wl.logits, wl.bias, wl.k)
    assert np.array_equal(idx_g, idx)
    y_ref = oracle.moe_output(wl.x, wl.bank, idx, w, decoder=shared_decoder(wl.bank))
    err, rms = assert_output(y.float().cpu().numpy().astype(np.float64), y_ref, f"per-route {name}")
    print(f"[per-route] {name}: every token, max_err={err:.3e} rms={rms:.3e}", flush=True)


# (H, I, E, k, T): tails (H/32 = 3, 5), k = E, several routes on one expert
@pytest.mark.parametrize("shape", [(96, 160, 8, 2, 5), (256, 64, 4, 4, 40), (640, 96, 16, 4, 33), (128, 4096, 6, 6, 3)],
                         ids=lambda s: "H%d_I%d_E%d_k%d_T%d" % s)
def test_per_route_edge_shapes(shape):
    H, I, E, k, T = shape
    wl = make_workload(replace(get_config("tiny"), name="per_route_edge", H=H, I=I, E=E, k=k, T=T), x_seed=41 + T)
    idx_g, w_g, y = _per_route(wl)
    idx, w = oracle.route_topk(wl.logits, wl.bias, wl.k)
    assert np.array_equal(idx_g, idx)
    y_ref = oracle.moe_output(wl.x, wl.bank, idx, w)
    assert_output(y.float().cpu().numpy().astype(np.float64), y_ref, f"per-route {shape}")


def test_per_route_deterministic():
    wl = make_workload("verify_t32", x_seed=5)
    a = _per_route(wl)[2]
    b = _per_route(wl)[2]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
