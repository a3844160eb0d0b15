"""Number formats read by the oracle: FP4 E2M1, FP8 E4M3FN, bf16 (test infrastructure).

The pages state only that the expert weights are NVFP4 in the checkpoint (page
"How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x faster on one GPU",
section "The model and the constraint").  The format definitions used here are
the public ones:
  * FP4 E2M1 (OCP Microscaling Formats spec v1.0): bit 3 sign, bits 2..1
    exponent with bias 1, bit 0 mantissa; exponent 0 is subnormal (m * 0.5).
  * FP8 E4M3FN (OCP 8-bit floating point spec): bit 7 sign, bits 6..3 exponent
    with bias 7, bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6);
    S.1111.111 is NaN, there are no infinities, the largest finite is 448.
  * NVFP4 block layout: one E4M3 scale per 16 consecutive elements along the
    reduction dimension and one fp32 global scale per matrix; element value =
    e2m1 * e4m3 * global.  Element 2i of a row is the low nibble of byte i.
"""

from __future__ import annotations

import numpy as np

# FP4 E2M1, indexed by the 4-bit code.  Codes 0..7 are the non-negative values
# {0, 0.5, 1, 1.5, 2, 3, 4, 6}; codes 8..15 are their negatives.
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def _e4m3_value(byte: int) -> float:
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3 = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """Value of every FP8 E4M3FN byte, float64[256] (NaN for 0x7F and 0xFF)."""
    return _E4M3.copy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> codes uint8 [..., 2n]; element 2i = low nibble of byte i."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """NVFP4 matrix [rows, cols/2] + scales [rows, cols/16] + global -> fp64 [rows, cols].

    W[r, c] = E2M1(code(r, c)) * E4M3(scales[r, c // 16]) * g, exact in fp64
    (at most 2 + 4 + 24 significant bits).
    """
    codes = unpack_nibbles(packed)
    rows, cols = codes.shape
    if scales.shape != (rows, cols // 16):
        raise ValueError(f"scale shape {scales.shape} does not match codes {codes.shape}")
    vals = E2M1_VALUES[codes]
    s = _E4M3[np.asarray(scales, dtype=np.uint8)]
    return vals * np.repeat(s, 16, axis=1) * float(g)
