"""The dense BF16 shared expert on the GPU (moe_shared_expert, through the C
ABI) against the oracle's fp64 evaluation, alone and beside a routed step on
a second stream (the routed output plus the shared one against the oracle's
routed output plus its shared one)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import DEV, assert_output, device_packed, device_weights, to_dev, x_bits
from moe_inputs import make_workload
from moe_inputs.generate import f64_to_bf16_bits

pytestmark = pytest.mark.gpu


def _weights(H, Is, seed):
    rng = np.random.default_rng(seed)
    wg = f64_to_bf16_bits(rng.standard_normal((Is, H)) / np.sqrt(H))
    wu = f64_to_bf16_bits(rng.standard_normal((Is, H)) / np.sqrt(H))
    wd = f64_to_bf16_bits(rng.standard_normal((H, Is)) / np.sqrt(Is))
    return wg, wu, wd


def _dev_bf16(bits):
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("T,H,Is", [(4, 2048, 512), (1, 2048, 512), (7, 512, 1024), (33, 1024, 512),
                                    (5, 4096, 512)])
def test_shared_expert(T, H, Is):
    rng = np.random.default_rng(T + H + Is)
    x = f64_to_bf16_bits(rng.standard_normal((T, H)))
    wg, wu, wd = _weights(H, Is, seed=T)
    y = sme.moe_shared_expert(x_bits(x), _dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd))
    y2 = sme.moe_shared_expert(x_bits(x), _dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))       # bitwise reproducible
    ref = oracle.shared_expert_output(x, wg, wu, wd)
    assert_output(y.float().cpu().numpy().astype(np.float64), ref, f"shared expert T={T} H={H} Is={Is}")


def test_beside_routed_step():
    """decode_t4: the routed step on the current stream and the shared expert
    on a second one (forked after the inputs are ready, joined before the
    sum); routed + shared against the oracle's routed + shared."""
    wl = make_workload("decode_t4")
    wg, wu, wd = _weights(wl.H, wl.I, seed=11)
    x = x_bits(wl.x)
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="packed")
    side = torch.cuda.Stream(DEV)
    main = torch.cuda.current_stream(DEV)
    gw, uw, dw = _dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd)
    torch.cuda.synchronize()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        ys = sme.moe_shared_expert(x, gw, uw, dw)
    st.run(x, to_dev(wl.logits), None, device_weights(wl.bank), packed=device_packed(wl.bank))
    main.wait_stream(side)
    y = (st.y.float() + ys.float()).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    idx, w = oracle.route_topk(wl.logits, None, wl.k)
    ref = oracle.moe_output(wl.x, wl.bank, idx, w) + oracle.shared_expert_output(wl.x, wg, wu, wd)
    assert_output(y, ref, "routed + shared, two streams")
