"""Test-side NVFP4 helpers written independently of the oracle.

Closed-form decoders computed from the bit fields, a nibble packer, builders
for hand-worked and random expert banks, and an exactly-rounded dense SwiGLU
FFN (math.fsum dot products).  Nothing here imports the oracle, so a mistake
in the oracle's tables, layout or arithmetic cannot cancel out.
"""

from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np


def e2m1_closed_form(code: int) -> float:
    """FP4 E2M1 from its fields: (-1)^s * (e == 0 ? m/2 : 2^(e-1) * (1 + m/2))."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e4m3_closed_form(byte: int) -> float:
    s = (byte >> 7) & 1
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 0xF and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes [..., 2n] (0..15) -> bytes [..., n]; element 2i -> low nibble of byte i."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def bf16_bits(v: float) -> int:
    """bf16 bits of a value exactly representable in bf16."""
    b = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, f"{v} is not exactly a bf16 value"
    return int(b >> 16)


def _matrix_from_spec(spec: dict, rows: int, cols: int):
    if "row_bytes" in spec:
        data = np.empty((rows, cols // 2), dtype=np.uint8)
        data[0::2] = int(spec["row_bytes"]["even"], 16)
        data[1::2] = int(spec["row_bytes"]["odd"], 16)
    else:
        data = np.full((rows, cols // 2), int(spec["byte"], 16), dtype=np.uint8)
    sc = np.array([int(s, 16) for s in spec["scales"]], dtype=np.uint8)
    assert sc.size == cols // 16
    scales = np.tile(sc, (rows, 1))
    return data, scales, np.float32(spec["g"])


def bank_from_case(case: dict):
    """Expert bank (oracle/GPU layout) from a hand-worked golden case."""
    H, I, E = case["H"], case["I"], case["E"]
    bank = SimpleNamespace(
        w_gate=np.zeros((E, I, H // 2), np.uint8), s_gate=np.zeros((E, I, H // 16), np.uint8),
        w_up=np.zeros((E, I, H // 2), np.uint8), s_up=np.zeros((E, I, H // 16), np.uint8),
        w_down=np.zeros((E, H, I // 2), np.uint8), s_down=np.zeros((E, H, I // 16), np.uint8),
        g_scale=np.zeros((E, 3), np.float32))
    for e, ex in enumerate(case["experts"]):
        bank.w_gate[e], bank.s_gate[e], bank.g_scale[e, 0] = _matrix_from_spec(ex["gate"], I, H)
        bank.w_up[e], bank.s_up[e], bank.g_scale[e, 1] = _matrix_from_spec(ex["up"], I, H)
        bank.w_down[e], bank.s_down[e], bank.g_scale[e, 2] = _matrix_from_spec(ex["down"], H, I)
    return bank


def x_from_case(case: dict) -> np.ndarray:
    T, H = case["T"], case["H"]
    x = np.empty((T, H), dtype=np.uint16)
    x[:, 0::2] = bf16_bits(case["x"]["even"])
    x[:, 1::2] = bf16_bits(case["x"]["odd"])
    return x


# A spread of finite e4m3 scale bytes (exponents 2^-5 .. 2^3, all mantissas).
_SCALE_BYTES = np.arange(0x10, 0x58, dtype=np.uint8)


def random_grid_bank(rng: np.random.Generator, E: int, H: int, I: int):
    """Random NVFP4 experts plus their exact fp64 matrices decoded in closed form.

    Returns (bank, dense) where dense[e] = (Wg [I,H], Wu [I,H], Wd [H,I]).
    """
    e2 = np.array([e2m1_closed_form(c) for c in range(16)])
    e4 = np.array([e4m3_closed_form(b) if b not in (0x7F, 0xFF) else 0.0 for b in range(256)])
    bank = SimpleNamespace(
        w_gate=np.zeros((E, I, H // 2), np.uint8), s_gate=np.zeros((E, I, H // 16), np.uint8),
        w_up=np.zeros((E, I, H // 2), np.uint8), s_up=np.zeros((E, I, H // 16), np.uint8),
        w_down=np.zeros((E, H, I // 2), np.uint8), s_down=np.zeros((E, H, I // 16), np.uint8),
        g_scale=np.zeros((E, 3), np.float32))
    dense = []
    for e in range(E):
        mats = []
        for m, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
            codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
            scales = rng.choice(_SCALE_BYTES, size=(rows, cols // 16))
            g = np.float32(rng.uniform(0.01, 0.2))
            W = e2[codes] * np.repeat(e4[scales], 16, axis=1) * float(g)
            name = ["gate", "up", "down"][m]
            getattr(bank, "w_" + name)[e] = pack_codes(codes)
            getattr(bank, "s_" + name)[e] = scales
            bank.g_scale[e, m] = g
            mats.append(W)
        dense.append(tuple(mats))
    return bank, dense


def _fdot(row, vec) -> float:
    return math.fsum(float(a) * float(b) for a, b in zip(row, vec))


def dense_swiglu_exact(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """W_down (SiLU(W_gate x) * (W_up x)) with exactly rounded dot products."""
    g = np.array([_fdot(r, x) for r in Wg])
    u = np.array([_fdot(r, x) for r in Wu])
    a = np.array([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
    return np.array([_fdot(r, a) for r in Wd])


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
