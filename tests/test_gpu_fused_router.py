"""moe_router_route_bucket (projection, selection and buckets in one call).

Through the C ABI: the fused call against moe_router_logits +
moe_route_bucket bit for bit on every output (logits, ids, weights, the six
bucket arrays), its counter back at 0 after every call, its logits within the
router bound of the oracle and its routing bit for bit the oracle's routing of
those logits; batches on both sides of the one-launch limit (16 tokens), both
workgroup sizes (512 and 1024 threads), H with one and two 16-byte pieces per
thread, E not a multiple of the rows per workgroup, k = E and k = 32; calls
back to back without a synchronisation between them; and a captured graph
replayed with changed inputs, each replay bit for bit its eager result.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import DEV, assert_buckets, assert_route, to_dev, x_bits
from test_gpu_router import _check_logits

pytestmark = pytest.mark.gpu


class _Outs:
    def __init__(self, T, E, k):
        self.logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        self.w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        self.b = sme.empty_buckets(T, E, k, DEV)

    def tensors(self):
        return [self.logits, self.idx, self.w.view(torch.int32), *self.b]


def _inputs(T, H, E, seed, with_bias):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)          # bf16 bits (truncated: any bf16 values)
    w = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if with_bias else None
    return xb, w, bias


def _fused(xd, wd, bd, k, counter, outs):
    sme.moe_router_route_bucket(xd, wd, bd, k, outs.logits, outs.idx, outs.w, outs.b, counter)


def _two_calls(xd, wd, bd, k, outs):
    sme.moe_router_logits(xd, wd, outs.logits)
    sme.moe_route_bucket(outs.logits, bd, k, outs.idx, outs.w, outs.b)


# (T, H, E, k, bias): one launch up to 16 tokens (512 threads when E <= 512
# and T <= 8, else 1024), two launches above
CASES = [
    (4, 2048, 512, 10, False), (1, 2048, 512, 10, True), (8, 2048, 512, 10, True), (12, 2048, 512, 10, False),
    (16, 2048, 1000, 8, True), (4, 4096, 512, 10, False), (5, 520, 64, 32, False), (3, 8, 5, 5, True),
    (7, 1024, 999, 1, False), (17, 2048, 512, 10, False), (40, 256, 100, 3, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_E%d_k%d_bias%d" % c)
def test_fused_router_matches_calls_and_oracle(case):
    T, H, E, k, with_bias = case
    xb, w, bias = _inputs(T, H, E, 500 + T + E, with_bias)
    xd, wd = x_bits(xb), to_dev(w)
    bd = None if bias is None else to_dev(bias)
    counter = torch.zeros(1, dtype=torch.int32, device=DEV)
    a, b = _Outs(T, E, k), _Outs(T, E, k)
    _fused(xd, wd, bd, k, counter, a)
    _two_calls(xd, wd, bd, k, b)
    torch.cuda.synchronize()
    assert int(counter.item()) == 0
    for ta, tb in zip(a.tensors(), b.tensors()):
        assert torch.equal(ta, tb)
    lg = a.logits.cpu().numpy()
    _check_logits(lg, xb, w)
    idx, wt = oracle.route_topk(lg, bias, k)
    g = {"idx": a.idx.cpu().numpy(), "w": a.w.cpu().numpy()}
    g.update({n: t.cpu().numpy() for n, t in zip(sme.Buckets._fields, a.b)})
    assert_route(g, idx, wt)
    assert_buckets(g, oracle.bucket_routes(idx, E))


def test_fused_router_back_to_back():
    """Ten calls on one stream with no synchronisation between them: each
    starts from the counter the previous one left at 0."""
    T, H, E, k = 4, 2048, 512, 10
    counter = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref = _Outs(T, E, k)
    outs = [_Outs(T, E, k) for _ in range(10)]
    ins = [_inputs(T, H, E, 900 + i, i % 2 == 0) for i in range(10)]
    dev_ins = [(x_bits(x), to_dev(w), None if b is None else to_dev(b)) for x, w, b in ins]
    for (xd, wd, bd), o in zip(dev_ins, outs):
        _fused(xd, wd, bd, k, counter, o)
    torch.cuda.synchronize()
    assert int(counter.item()) == 0
    for (xd, wd, bd), o in zip(dev_ins, outs):
        _two_calls(xd, wd, bd, k, ref)
        torch.cuda.synchronize()
        for ta, tb in zip(o.tensors(), ref.tensors()):
            assert torch.equal(ta, tb)


def test_fused_router_graph_replays():
    """Captured once; replayed with inputs A, B, A (eager work and a
    synchronisation between replays); every replay equals the eager call on
    its inputs bit for bit, and the counter is 0 after each."""
    T, H, E, k = 4, 2048, 512, 10
    A = _inputs(T, H, E, 71, True)
    B = _inputs(T, H, E, 72, True)
    x_s, w_s = x_bits(A[0]), to_dev(A[1])
    b_s = to_dev(A[2])
    counter = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = _Outs(T, E, k)
    _fused(x_s, w_s, b_s, k, counter, o)           # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fused(x_s, w_s, b_s, k, counter, o)
    torch.cuda.synchronize()
    for rep, (xb, w, bias) in enumerate([A, B, A]):
        x_s.copy_(x_bits(xb))
        w_s.copy_(to_dev(w))
        b_s.copy_(to_dev(bias))
        junk = torch.randn(1024, device=DEV).sum()
        g.replay()
        torch.cuda.synchronize()
        assert int(counter.item()) == 0, rep
        ref = _Outs(T, E, k)
        c2 = torch.zeros(1, dtype=torch.int32, device=DEV)
        _fused(x_bits(xb), to_dev(w), to_dev(bias), k, c2, ref)
        torch.cuda.synchronize()
        for ta, tb in zip(o.tensors(), ref.tensors()):
            assert torch.equal(ta, tb), rep
        del junk
