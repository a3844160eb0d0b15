"""NVFP4 encoder: float weights -> (e2m1 codes, e4m3 block scales, fp32 global).

Storage format (public format definitions; the pages only say the expert
weights are NVFP4 in the checkpoint):
  * value elements are FP4 E2M1 (OCP Microscaling spec): sign bit 3, exponent
    bits 2..1 (bias 1), mantissa bit 0; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6};
  * one FP8 E4M3FN scale (OCP 8-bit float spec: bias 7, no infinities,
    max 448) per 16 consecutive elements along the reduction dimension;
  * one fp32 global scale per matrix; element = e2m1 * e4m3 * global.
  * packing: element 2i of a row sits in the low nibble of byte i, element
    2i+1 in the high nibble.

Encoding recipe (a reading; the pages give none): per matrix
g = amax / (6 * 448) rounded to fp32 (g = 1 when amax = 0); per block
s = e4m3_RNE(amax_blk / (6 g)); codes = e2m1_RNE(w / (s g)) with ties to the
even code and saturation at +-6; s = 0 gives all-zero codes.

This module only encodes.  It holds no decoder used by anything else.
"""

from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0

# Decision thresholds between consecutive e2m1 magnitudes
# 0 | 0.5 | 1 | 1.5 | 2 | 3 | 4 | 6 are the midpoints below.  A value exactly on
# a midpoint goes to the neighbour whose code is even (round half to even on
# the code): strict ">" where the lower neighbour is even, ">=" where the
# upper one is.
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_MID_UPPER_EVEN = (False, True, False, True, False, True, False)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest FP4 E2M1 code (uint8 in 0..15).

    Round-to-nearest, ties to the even code, saturating at +-6.  Values whose
    magnitude rounds to zero get code 0 (no negative-zero codes).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    mag = np.zeros(v.shape, dtype=np.uint8)
    for m, up in zip(_E2M1_MID, _E2M1_MID_UPPER_EVEN):
        mag += (a >= m) if up else (a > m)
    sign = ((v < 0) & (mag > 0)).astype(np.uint8) << 3
    return mag | sign


def encode_e4m3(v: np.ndarray):
    """Round non-negative float64 values to FP8 E4M3FN, RNE, saturating at 448.

    Returns (bytes uint8, rounded values float64).  The rounded values are
    produced by the rounding itself (q * quantum), not by decoding the bytes.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3 scale encoder expects finite non-negative values")
    v = np.minimum(v, E4M3_MAX)
    out_val = np.zeros_like(v)
    out_byte = np.zeros(v.shape, dtype=np.uint8)
    nz = v > 0
    vv = v[nz]
    # binade exponent, clamped to the smallest normal binade (2^-6); below it
    # the quantum stays 2^-9 (subnormals).
    e = np.floor(np.log2(vv))
    # guard against log2 rounding at exact powers of two
    e = np.where(np.exp2(e) > vv, e - 1, e)
    e = np.where(np.exp2(e + 1) <= vv, e + 1, e)
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3)
    q = np.rint(vv / quantum)            # numpy rint is round-half-to-even
    val = q * quantum
    val = np.minimum(val, E4M3_MAX)
    # bytes
    byte = np.zeros(vv.shape, dtype=np.int64)
    sub = val < 2.0 ** -6
    byte[sub] = np.rint(val[sub] / 2.0 ** -9).astype(np.int64)          # 0..7
    nrm = ~sub & (val > 0)
    ve = np.floor(np.log2(val[nrm]))
    ve = np.where(np.exp2(ve) > val[nrm], ve - 1, ve)
    mant = np.rint((val[nrm] / np.exp2(ve) - 1.0) * 8).astype(np.int64)  # 0..7
    byte[nrm] = ((ve.astype(np.int64) + 7) << 3) | mant
    out_val[nz] = val
    out_byte[nz] = byte.astype(np.uint8)
    return out_byte, out_val


def encode_nvfp4(w: np.ndarray):
    """Encode matrices [..., rows, cols] (cols % 16 == 0) to NVFP4.

    One global scale per leading index (per matrix).  Returns
    (packed codes uint8 [..., rows, cols/2], scales uint8 [..., rows, cols/16],
    global scale float32 [...]).
    """
    w = np.asarray(w)
    if w.ndim < 2 or w.shape[-1] % 16 != 0:
        raise ValueError("need [..., rows, cols] with cols a multiple of 16")
    lead = w.shape[:-2]
    rows, cols = w.shape[-2:]
    w64 = w.astype(np.float64)
    amax = np.abs(w64).reshape(lead + (-1,)).max(axis=-1) if w64.size else np.zeros(lead)
    g = np.where(amax > 0, amax / (E2M1_MAX * E4M3_MAX), 1.0).astype(np.float32)
    g64 = g.astype(np.float64)[..., None, None, None]
    blocks = w64.reshape(lead + (rows, cols // 16, 16))
    bmax = np.abs(blocks).max(axis=-1, keepdims=True)
    s_byte, s_val = encode_e4m3(bmax / (E2M1_MAX * g64))
    denom = s_val * g64
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(denom > 0, blocks / np.where(denom > 0, denom, 1.0), 0.0)
    codes = encode_e2m1(ratio).reshape(lead + (rows, cols))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = s_byte.reshape(lead + (rows, cols // 16)).astype(np.uint8)
    return packed, scales, g
