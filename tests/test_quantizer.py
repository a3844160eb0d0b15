"""The NVFP4 encoder that makes the synthetic expert weights.

Pinned against the oracle's decoder (itself pinned to the format specs):
per-element error within half an e2m1 step of the block's scale, saturation,
zero blocks, exact round trips of grid values, and e4m3 rounding.
"""

import numpy as np

import oracle
from moe_inputs import encode_e2m1, encode_e4m3, encode_nvfp4

_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _half_step(a):
    # half the gap to the next e2m1 magnitude above |a|
    a = np.minimum(np.abs(a), 6.0)
    return np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))


def test_e2m1_grid_round_trip():
    v = np.concatenate([_GRID, -_GRID[1:]])
    codes = encode_e2m1(v)
    assert np.array_equal(oracle.E2M1_VALUES[codes], v)


def test_e2m1_ties_to_even_and_saturation():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.25, -5.0])
    got = oracle.E2M1_VALUES[encode_e2m1(mids)]
    assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.0, -4.0]


def test_e4m3_round_trip_and_rne():
    tab = oracle.e4m3_table()
    finite = np.array([b for b in range(0x7F) if np.isfinite(tab[b])])
    byte, val = encode_e4m3(tab[finite])
    assert np.array_equal(byte, finite.astype(np.uint8))
    assert np.array_equal(val, tab[finite])
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even mantissa 0x38
    b, v = encode_e4m3(np.array([1.0625, 1.1875, 500.0, 2.0 ** -10, 3 * 2.0 ** -11]))
    assert b.tolist() == [0x38, 0x3A, 0x7E, 0x00, 0x01]


def test_block_error_bound_and_layout():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3, 24, 64)).astype(np.float32) * np.float32(0.05)
    w[1, 5, 16:32] = 0.0        # an all-zero block
    w[2, 0, 0] = 3.0            # a dominant element
    packed, scales, g = encode_nvfp4(w)
    assert packed.shape == (3, 24, 32) and scales.shape == (3, 24, 4) and g.shape == (3,)
    for m in range(3):
        deq = oracle.dequant_nvfp4(packed[m], scales[m], float(g[m]))
        s = oracle.e4m3_table()[scales[m]]
        sg = np.repeat(s, 16, axis=1) * float(g[m])
        ratio = np.where(sg > 0, w[m] / np.where(sg > 0, sg, 1), 0)
        err = np.abs(deq - w[m].astype(np.float64))
        bound = np.maximum(_half_step(ratio), np.abs(ratio) - 6.0) * sg
        assert np.all(err <= bound * (1 + 1e-12) + 1e-300)
        assert np.all(np.abs(deq) <= 6 * sg + 1e-300)
    assert np.all(scales[1, 5, 1] == 0)
    assert np.all(oracle.unpack_nibbles(packed[1, 5:6])[0, 16:32] == 0)
    # amax element maps to +-6 * scale * g with scale <= 448
    assert oracle.dequant_nvfp4(packed[2], scales[2], float(g[2]))[0, 0] > 2.5


def test_zero_matrix():
    packed, scales, g = encode_nvfp4(np.zeros((1, 4, 32), np.float32))
    assert np.all(packed == 0) and np.all(scales == 0) and g[0] == 1.0
