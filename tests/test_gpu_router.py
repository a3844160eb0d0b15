"""GPU parity of the router projection (moe_router_logits) against the oracle.

Both sides form fp64 sums of exact products and round once to fp32, in
different orders; a logit may therefore differ by one fp32 ulp, and only when
the exact sum lies within the fp64 accumulation error of a rounding boundary
(bound: ulp + 2 * H * 2^-53 * sum |x w|).  Almost every logit is identical;
the routing chosen from the GPU logits is checked against the oracle's
routing of the same logits bit for bit, and a step from tokens (projection,
routing, expert FFN) against the oracle end to end.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import (DEV, assert_buckets, assert_output, assert_route, collect, device_packed, device_weights,
                         shared_decoder, x_bits)
from moe_inputs import make_workload

pytestmark = pytest.mark.gpu


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # round to nearest even


def _check_logits(got, x_u16, w):
    ref = oracle.router_logits(x_u16, w)
    xv = oracle.bf16_bits_to_f64(x_u16)
    absum = np.abs(xv) @ np.abs(w.astype(np.float64)).T
    ulp = np.abs(np.spacing(ref.astype(np.float32))).astype(np.float64)
    bound = ulp + 2.0 * x_u16.shape[1] * 2.0 ** -53 * absum
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(diff <= bound), float(np.max(diff / bound))
    assert np.mean(got == ref) >= 0.999, np.mean(got == ref)
    return ref


# (T, H, E): decode, one token, ragged token groups, small and odd sizes, the
# largest row, both sides of the 64- and 1024-token switches between the three
# kernels (a K tail at H = 520, ragged token and expert tiles), a prefill chunk
ROUTER_SHAPES = [(4, 2048, 512), (1, 2048, 512), (33, 2048, 512), (5, 256, 100), (9, 8, 3), (17, 4096, 64),
                 (3, 520, 1000), (64, 2048, 512), (65, 1024, 40), (100, 4096, 33), (1023, 256, 70),
                 (1024, 520, 130), (1500, 64, 1000), (4096, 2048, 512)]


@pytest.mark.parametrize("shape", ROUTER_SHAPES, ids=lambda s: "T%d_H%d_E%d" % s)
def test_router_logits(shape):
    T, H, E = shape
    rng = np.random.default_rng(300 + T + H + E)
    x = _bf16_bits(rng.standard_normal((T, H)))
    w = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    got = sme.moe_router_logits(x_bits(x), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    _check_logits(got.cpu().numpy(), x, w)


@pytest.mark.parametrize("name", ["tiny", "decode_t4", "verify_t32"])
def test_step_from_tokens(name):
    """Projection, routing and expert FFN from the workload's tokens and router
    weights: the logits against the oracle, then the routing of those logits
    and the output against the oracle bit for bit / within 2e-2 rms."""
    wl = make_workload(name)
    xd = x_bits(wl.x)
    logits = sme.moe_router_logits(xd, torch.from_numpy(wl.w_router).to(DEV))
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    _check_logits(lg, wl.x, wl.w_router)
    bias = None if wl.bias is None else torch.from_numpy(wl.bias).to(DEV)
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="packed")
    st.run(xd, logits, bias, device_weights(wl.bank), packed=device_packed(wl.bank))
    torch.cuda.synchronize()
    g = collect(st)
    idx, w = oracle.route_topk(lg, wl.bias, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, oracle.bucket_routes(idx, wl.E))
    y = oracle.moe_output(wl.x, wl.bank, idx, w, decoder=shared_decoder(wl.bank))
    assert_output(g["y"], y, f"{name} from tokens")
