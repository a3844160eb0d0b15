"""moe_step_noalloc (static scratch, no workspace argument) against moe_step.

Through the C ABI: two calls in a row (128 tokens, then 4), each
compared with moe_step (its own workspace) bit for bit on every output and
with the oracle (bit-exact ids and buckets, gate weights within 1e-6, the
output within 2e-2 * rms plus half a bf16 ulp); the packed variant too; a
batch whose workspace exceeds the scratch is refused before any launch.
"""

import numpy as np
import pytest
import torch

import sparse_moe_expert_amd as sme
from gpu_harness import (DEV, assert_buckets, assert_output, assert_route, collect, device_packed, device_weights,
                         oracle_all, to_dev, x_bits)
from moe_inputs import make_workload

pytestmark = pytest.mark.gpu


def _noalloc_outputs(wl, packed):
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="step")
    st.workspace = None                    # the no-allocation call takes none
    sme.moe_step_noalloc(x_bits(wl.x), to_dev(wl.logits), None if wl.bias is None else to_dev(wl.bias),
                         device_weights(wl.bank), wl.k, st.topk_idx, st.topk_w, st.buckets, st.y,
                         packed=packed)
    return st


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_step_twice(packed):
    # 128 tokens (matrix-core tiles, per-route o in the scratch, combine), then 4
    runs = [make_workload("decode_t4", T=128, x_seed=21), make_workload("decode_t4", x_seed=22)]
    assert runs[1].T < runs[0].T
    for wl in runs:
        print(f"[noalloc] T={wl.T} packed={packed}", flush=True)
        pk = device_packed(wl.bank) if packed else None
        a = _noalloc_outputs(wl, pk)
        ref = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="packed" if packed else "step")
        ref.run(x_bits(wl.x), to_dev(wl.logits), None if wl.bias is None else to_dev(wl.bias),
                device_weights(wl.bank), packed=pk)
        torch.cuda.synchronize()
        assert torch.equal(a.topk_idx, ref.topk_idx)
        assert torch.equal(a.topk_w.view(torch.int32), ref.topk_w.view(torch.int32))
        for ta, tb in zip(a.buckets, ref.buckets):
            assert torch.equal(ta, tb)
        assert torch.equal(a.y.view(torch.int16), ref.y.view(torch.int16))
        g = collect(a)
        idx, w, b, y = oracle_all(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
        assert_route(g, idx, w)
        assert_buckets(g, b)
        err, rms = assert_output(g["y"], y, f"noalloc T={wl.T}")
        print(f"[noalloc] T={wl.T} packed={packed}: bit for bit moe_step, max_err={err:.3e} rms={rms:.3e}",
              flush=True)


def test_noalloc_refuses_batches_beyond_scratch():
    wl = make_workload("decode_t4", T=164, x_seed=23)
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="step")
    st.y.fill_(1.0)
    with pytest.raises(sme.MoeError) as ei:
        sme.moe_step_noalloc(x_bits(wl.x), to_dev(wl.logits), None, device_weights(wl.bank), wl.k,
                             st.topk_idx, st.topk_w, st.buckets, st.y)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(st.y == 1.0)
