"""Pins of the oracle's dense shared expert (CPU).

1. Closed form: constant weights and a constant token give
   y = Is * c_d * SiLU(H * c_g * v) * (H * c_u * v) in every output row.
2. Reduction to the routed oracle: a routed expert with k = 1 is the same
   SwiGLU chain with gate weight 1; NVFP4 weights with global scale 1 are
   exact in bf16 (e2m1 x e4m3 has at most 6 significant bits), so the shared
   expert on those bf16 weights must equal moe_output with one expert, to the
   last bit of the fp64 arithmetic.
3. Planted mistakes (gate and up swapped, SiLU left out) fail the reduction.
"""

import numpy as np

import oracle
from moe_inputs.generate import f64_to_bf16_bits


def _bf16(v):
    return f64_to_bf16_bits(np.asarray(v, dtype=np.float64))


def test_closed_form():
    T, H, Is = 3, 64, 32
    cg, cu, cd, v = 0.015625, -0.03125, 0.0625, 0.5          # exact in bf16
    x = _bf16(np.full((T, H), v))
    y = oracle.shared_expert_output(x, _bf16(np.full((Is, H), cg)), _bf16(np.full((Is, H), cu)),
                                    _bf16(np.full((H, Is), cd)))
    g, u = H * cg * v, H * cu * v
    ref = Is * cd * (g / (1.0 + np.exp(-g))) * u
    assert y.shape == (T, H)
    assert np.allclose(y, ref, rtol=0, atol=1e-15)


def _bank_one_expert(H, Is, seed):
    """One NVFP4 expert with global scales 1 (its values are then exact in bf16)."""
    from moe_inputs.nvfp4_encode import encode_nvfp4
    from types import SimpleNamespace
    rng = np.random.default_rng(seed)
    mats = {}
    for name, shape in (("gate", (Is, H)), ("up", (Is, H)), ("down", (H, Is))):
        codes, scales, g = encode_nvfp4(rng.standard_normal(shape) * 50.0)
        mats[name] = (codes, scales)
    g1 = np.ones((1, 3), dtype=np.float32)
    return SimpleNamespace(w_gate=mats["gate"][0][None], s_gate=mats["gate"][1][None],
                           w_up=mats["up"][0][None], s_up=mats["up"][1][None],
                           w_down=mats["down"][0][None], s_down=mats["down"][1][None], g_scale=g1)


def test_reduces_to_routed_expert():
    H, Is, T = 64, 32, 4
    bank = _bank_one_expert(H, Is, seed=7)
    dec = oracle.ExpertDecoder(bank)
    wg, wu, wd = dec.matrices(0)
    for w in (wg, wu, wd):                                    # exact in bf16
        assert np.array_equal(oracle.bf16_bits_to_f64(_bf16(w)), w)
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((T, H)))
    idx = np.zeros((T, 1), dtype=np.int32)
    w1 = np.ones((T, 1), dtype=np.float64)
    routed = oracle.moe_output(x, bank, idx, w1)
    shared = oracle.shared_expert_output(x, _bf16(wg), _bf16(wu), _bf16(wd))
    assert np.array_equal(shared, routed)


def test_planted_mistakes_fail():
    """Plausible slips in a shared-expert evaluation (gate and up swapped,
    SiLU left out) differ from the routed oracle's chain."""
    H, Is, T = 64, 32, 4
    bank = _bank_one_expert(H, Is, seed=8)
    wg, wu, wd = oracle.ExpertDecoder(bank).matrices(0)
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((T, H)))
    routed = oracle.moe_output(x, bank, np.zeros((T, 1), np.int32), np.ones((T, 1)))
    swapped = oracle.shared_expert_output(x, _bf16(wu), _bf16(wg), _bf16(wd))
    assert not np.allclose(swapped, routed)
    xt = oracle.bf16_bits_to_f64(x)
    no_silu = np.stack([wd @ ((wg @ xt[t]) * (wu @ xt[t])) for t in range(T)])
    assert not np.allclose(no_silu, routed)
    assert np.array_equal(oracle.shared_expert_output(x, _bf16(wg), _bf16(wu), _bf16(wd)), routed)
