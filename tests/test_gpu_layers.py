"""Chained layers on the GPU against the oracle, layer by layer.

L routed-MoE layers, each with its own router weights and experts: per layer
the router projection (moe_router_logits) and one step (moe_step_packed) on
that layer's input; layer l+1's input is layer l's input plus its bf16
output (a residual stream, the add done by torch).
Each layer is checked against the oracle on the GPU's own input to it (the
logits within the router bound, the routing of those logits bit for bit, the
output within 2e-2 rms), so that one layer's rounding does not move the next
layer's reference.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import DEV, assert_buckets, assert_output, assert_route, collect, device_packed, device_weights, x_bits
from moe_inputs import make_workload
from test_gpu_router import _check_logits

pytestmark = pytest.mark.gpu


def _layer_bank(bank, shift):
    """The experts of another layer: bank 0's experts rolled by `shift`."""
    from types import SimpleNamespace
    return SimpleNamespace(**{k: (np.roll(v, shift, axis=0) if isinstance(v, np.ndarray) else v)
                              for k, v in vars(bank).items()})


@pytest.mark.parametrize("name,layers", [("tiny", 3), ("decode_t4", 2), ("verify_t32", 2)])
def test_chained_layers(name, layers):
    base = make_workload(name)
    x = base.x
    xd = x_bits(x)
    for l in range(layers):
        lw = make_workload(name, seed=base.cfg.seed + 100 + l, with_bank=False)
        bank = _layer_bank(base.bank, 67 * l)
        logits = sme.moe_router_logits(xd, torch.from_numpy(lw.w_router).to(DEV))
        st = sme.MoeStep(base.T, base.H, base.I, base.E, base.k, DEV, path="packed")
        bias = None if lw.bias is None else torch.from_numpy(lw.bias).to(DEV)
        st.run(xd, logits, bias, device_weights(bank), packed=device_packed(bank))
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        _check_logits(lg, x, lw.w_router)
        g = collect(st)
        idx, w = oracle.route_topk(lg, lw.bias, base.k)
        assert_route(g, idx, w)
        assert_buckets(g, oracle.bucket_routes(idx, base.E))
        # every token; this layer's experts decoded once (dropped after the layer)
        y = oracle.moe_output(x, bank, idx, w, decoder=oracle.ExpertDecoder(bank, cache=base.E))
        assert_output(g["y"], y, f"{name} layer {l}")
        # the next layer's input: this layer's input plus its bf16 output (a
        # residual stream; without it the outputs shrink until routing ties)
        xd = torch.add(xd.view(torch.bfloat16), st.y)
        x = xd.view(torch.int16).cpu().numpy().view(np.uint16)
