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


def _custom(T, H, I, E, k):
    from dataclasses import replace
    from moe_inputs.configs import get_config
    return make_workload(replace(get_config("tiny"), name="step_shared", T=T, H=H, I=I, E=E, k=k), x_seed=T + E)


# (workload, Is, packed): which of the shared expert's halves ride along in
# the step's launches - the small step (up to 40 routes at H = 2048):
# gate/up rows in the selection launch, down rows in the last waves of the
# route-slot down/unroute (decode_t4: 4 rows per workgroup, one chunk per
# lane; T=1, Is=1024: two chunks per lane; I=256: 8 rows per workgroup, E=64;
# I=1024: 2 rows per workgroup, 40 routes; T=8, Is=1024: the shared h at the
# 16 KB limit and the down rows' token loop); T=3, Is=2048 (four chunks per
# down row): the three-kernel step, down on its own.  T=12: both in the
# three-kernel step (1024-thread routing workgroup, two chunks per down row);
# verify_t32: gate/up on its own (routing takes several kernels), down in
# the row-dot kernel; decode_t256_zipf packed: down on its own (no row-dot
# kernel), standard layout: down beside the sorted row-dot experts; H=512,
# Is=2048: gate/up with one chunk per row, down on its own (four chunks).
STEP_SHARED_CASES = [
    ("decode_t4", 512, True), ((1, 2048, 512, 512, 10), 1024, True), ((4, 2048, 256, 64, 8), 512, False),
    ((2, 2048, 1024, 128, 20), 512, True), ((8, 2048, 512, 512, 5), 1024, True),
    ((3, 2048, 512, 512, 10), 2048, True),
    ((12, 2048, 512, 512, 10), 1024, True), ("verify_t32", 512, True),
    ("decode_t256_zipf", 512, True), ("decode_t256_zipf", 512, False), ((5, 512, 256, 64, 4), 2048, False),
]


@pytest.mark.parametrize("case", STEP_SHARED_CASES,
                         ids=lambda c: "%s_Is%d_%s" % (c[0] if isinstance(c[0], str) else "T%d_H%d_I%d_E%d_k%d" % c[0],
                                                       c[1], "packed" if c[2] else "std"))
def test_step_shared(case):
    """moe_step_shared: y bit for bit moe_step(_packed)'s, y_shared bit for
    bit moe_shared_expert's and within tolerance of the oracle's."""
    name, Is, packed = case
    wl = make_workload(name) if isinstance(name, str) else _custom(*name)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    wg, wu, wd = _weights(H, Is, seed=T + Is)
    gw, uw, dw = _dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd)
    x = x_bits(wl.x)
    logits = to_dev(wl.logits)
    bias = None if wl.bias is None else to_dev(wl.bias)
    W = device_weights(wl.bank)
    pk = device_packed(wl.bank) if packed else None
    path = "packed" if packed else "step"
    ref_step = sme.MoeStep(T, H, I, E, k, DEV, path=path)
    ref_step.run(x, logits, bias, W, packed=pk)
    ref_shared = sme.moe_shared_expert(x, gw, uw, dw)
    st = sme.MoeStep(T, H, I, E, k, DEV, path=path)
    ys = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(16, sme.load_library().moe_shared_expert_workspace_size(T, H, Is)), dtype=torch.uint8,
                     device=DEV)
    for _ in range(2):   # a second call over the same buffers gives the same bits
        sme.moe_step_shared(x, logits, bias, W, k, st.topk_idx, st.topk_w, st.buckets, st.workspace, st.y,
                            (gw, uw, dw), ys, ws, packed=pk)
        torch.cuda.synchronize()
        assert torch.equal(st.topk_idx, ref_step.topk_idx)
        assert torch.equal(st.y.view(torch.int16), ref_step.y.view(torch.int16))
        assert torch.equal(ys.view(torch.int16), ref_shared.view(torch.int16))
    ref = oracle.shared_expert_output(wl.x, wg, wu, wd)
    assert_output(ys.float().cpu().numpy().astype(np.float64), ref, f"moe_step_shared {case}")


def test_step_shared_graph_replays():
    """moe_step_shared captured in a graph (decode_t4, both halves riding
    along): three replays with inputs A, B, A and eager work between them,
    each against the eager result for its input, bit for bit."""
    wl = make_workload("decode_t4")
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    wg, wu, wd = _weights(H, I, seed=3)
    sh = (_dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd))
    W = device_weights(wl.bank)
    pk = device_packed(wl.bank)
    xa, xb = x_bits(wl.x), x_bits(make_workload("decode_t4", x_seed=77).x)
    la, lb = to_dev(wl.logits), to_dev(np.roll(wl.logits, 5, axis=1).copy())
    x_in, l_in = xa.clone(), la.clone()
    st = sme.MoeStep(T, H, I, E, k, DEV, path="packed")
    ys = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(16, sme.load_library().moe_shared_expert_workspace_size(T, H, I)), dtype=torch.uint8,
                     device=DEV)

    def call():
        sme.moe_step_shared(x_in, l_in, None, W, k, st.topk_idx, st.topk_w, st.buckets, st.workspace, st.y, sh, ys,
                            ws, packed=pk)

    eager = {}
    for name, xv, lv in (("A", xa, la), ("B", xb, lb)):
        x_in.copy_(xv)
        l_in.copy_(lv)
        call()
        torch.cuda.synchronize()
        eager[name] = (st.y.clone(), ys.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for name, xv, lv in (("A", xa, la), ("B", xb, lb), ("A", xa, la)):
        x_in.copy_(xv)
        l_in.copy_(lv)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.y.view(torch.int16), eager[name][0].view(torch.int16)), name
        assert torch.equal(ys.view(torch.int16), eager[name][1].view(torch.int16)), name
        torch.add(ys, 1.0)   # eager work between replays
        torch.cuda.synchronize()


def test_step_shared_small_guard_regions():
    """The small step with the shared rows riding along (decode_t4, Is=1024):
    canaries around y_shared and the shared workspace stay untouched, and
    both outputs match the separate calls bit for bit."""
    wl = make_workload("decode_t4", x_seed=23)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    Is = 1024
    wg, wu, wd = _weights(H, Is, seed=29)
    gw, uw, dw = _dev_bf16(wg), _dev_bf16(wu), _dev_bf16(wd)
    x, logits, W = x_bits(wl.x), to_dev(wl.logits), device_weights(wl.bank)
    ref_step = sme.MoeStep(T, H, I, E, k, DEV, path="step")
    ref_step.run(x, logits, None, W)
    ref_shared = sme.moe_shared_expert(x, gw, uw, dw)
    ws_bytes = sme.load_library().moe_shared_expert_workspace_size(T, H, Is)
    big_ws = torch.full((ws_bytes + 512,), 0xA5, dtype=torch.uint8, device=DEV)
    big_ys = torch.full((T + 2, H), 3.0, dtype=torch.bfloat16, device=DEV)
    st = sme.MoeStep(T, H, I, E, k, DEV, path="step")
    sme.moe_step_shared(x, logits, None, W, k, st.topk_idx, st.topk_w, st.buckets, st.workspace, st.y,
                        (gw, uw, dw), big_ys[1: T + 1], big_ws[256: 256 + ws_bytes])
    torch.cuda.synchronize()
    assert torch.all(big_ws[:256] == 0xA5) and torch.all(big_ws[256 + ws_bytes:] == 0xA5)
    assert torch.all(big_ys[0] == 3.0) and torch.all(big_ys[T + 1] == 3.0)
    assert torch.equal(st.y.view(torch.int16), ref_step.y.view(torch.int16))
    assert torch.equal(big_ys[1: T + 1].view(torch.int16), ref_shared.view(torch.int16))
