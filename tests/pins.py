"""Pins that tie the oracle to facts outside itself.

Each check raises AssertionError on failure.  They are called by the pin tests
and, with a mistake planted in the oracle, by the mutation tests (which expect
them to fail).  Sources of truth: public format specs (golden JSON), values
worked by hand (golden JSON), closed forms, brute-force enumeration, library
routines (torch's float8_e4m3fn and bfloat16 casts, numpy's stable argsort and
lexsort), and exactly rounded (math.fsum) dense FFNs built from test-side
closed-form decoders.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

import oracle
from nvfp4_testlib import (
    bank_from_case,
    bf16_values,
    dense_swiglu_exact,
    e2m1_closed_form,
    random_grid_bank,
    x_from_case,
)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ev(expr) -> float:
    return float(eval(str(expr), {"math": math, "__builtins__": {}}))


# ---------------------------------------------------------------- formats (P1-P3)

def check_e2m1():
    g = load_golden("e2m1_ocp_mx.json")["code_to_value"]
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = oracle.unpack_nibbles(packed)[0]
    assert codes.shape == (512,)
    # byte b holds code b & 15 at even position, b >> 4 at odd position
    assert np.array_equal(codes[0::2], np.arange(256) & 15)
    assert np.array_equal(codes[1::2], np.arange(256) >> 4)
    for c in range(16):
        v = oracle.E2M1_VALUES[c]
        assert v == g[str(c)], (c, v)
        assert v == e2m1_closed_form(c), (c, v)
        assert math.copysign(1.0, v) == math.copysign(1.0, g[str(c)])


def check_e4m3():
    import torch
    tab = oracle.e4m3_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], lib[~nan])
    gold = load_golden("e4m3_ocp_fp8.json")
    for b, expr in gold["byte_to_value"].items():
        v = tab[int(b, 16)]
        assert v == _ev(expr) and math.copysign(1, v) == math.copysign(1, _ev(expr)), (b, v)
    for b in gold["nan_bytes"]:
        assert math.isnan(tab[int(b, 16)])


def check_products_exact_in_bf16():
    """Every e2m1 x finite e4m3 product survives a round trip through bf16."""
    import torch
    e2 = oracle.E2M1_VALUES
    e4 = oracle.e4m3_table()
    prods = (e2[:, None] * e4[None, :])
    prods = prods[np.isfinite(prods)]
    t = torch.from_numpy(prods)
    back = t.to(torch.bfloat16).double().numpy()
    assert np.array_equal(back, prods)


def check_dequant_layout():
    """dequant_nvfp4 against the closed form on random codes and scales."""
    rng = np.random.default_rng(5)
    bank, dense = random_grid_bank(rng, 2, 64, 32)
    for e in range(2):
        for m, name in enumerate(["gate", "up", "down"]):
            W = oracle.dequant_nvfp4(getattr(bank, "w_" + name)[e], getattr(bank, "s_" + name)[e],
                                     float(bank.g_scale[e, m]))
            assert np.array_equal(W, dense[e][m])


# ---------------------------------------------------------------- routing (P5-P7)

def check_routing_golden():
    for case in load_golden("routing_hand_worked.json")["cases"]:
        logits = np.array(case["logits"], dtype=np.float32)
        bias = None if case["bias"] is None else np.array(case["bias"], dtype=np.float32)
        idx, w = oracle.route_topk(logits, bias, case["k"])
        assert idx.tolist() == case["idx"], (case["name"], idx.tolist())
        exp = np.array([[_ev(v) for v in row] for row in case["w"]])
        assert np.max(np.abs(w - exp)) <= case["w_tol"], (case["name"], w, exp)


def _bruteforce_set(z, k):
    E = len(z)
    valid = []
    for A in itertools.combinations(range(E), k):
        rest = [z[e] for e in range(E) if e not in A]
        if not rest or min(z[e] for e in A) >= max(rest):
            valid.append(A)
    return min(valid)


def check_topk_bruteforce(seed: int = 0, cases: int = 400):
    rng = np.random.default_rng(seed)
    vals = np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32)
    for _ in range(cases):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        z = rng.choice(vals, size=E).astype(np.float32)
        if rng.random() < 0.3:
            z = rng.standard_normal(E).astype(np.float32)
        idx, _ = oracle.route_topk(z[None, :], None, k)
        sel = [int(e) for e in idx[0]]
        assert tuple(sorted(sel)) == _bruteforce_set([float(v) for v in z], k), (z, k, sel)
        for a, b in zip(sel, sel[1:]):
            assert z[a] > z[b] or (z[a] == z[b] and a < b), (z, sel)
        ref = np.argsort(-z.astype(np.float64), kind="stable")[:k]
        assert sel == ref.tolist(), (z, sel, ref)


def check_weight_invariants(seed: int = 1):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 5))
        logits = (rng.standard_normal((T, E)) * rng.uniform(0.1, 8)).astype(np.float32)
        idx, w = oracle.route_topk(logits, None, k)
        for t in range(T):
            assert abs(w[t].sum() - 1.0) <= k * 1e-15 + 1e-15, w[t].sum()
            assert np.all(np.diff(w[t]) <= 0), w[t]
            z = logits[t].astype(np.float64)[idx[t]]
            direct = np.exp(z - z.max()) / np.exp(z - z.max()).sum()   # softmax over the set
            assert np.allclose(w[t], direct, rtol=1e-12, atol=0), (w[t], direct)


# ---------------------------------------------------------------- buckets (P15)

def check_buckets(seed: int = 2):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        E = int(rng.integers(1, 70))
        k = int(rng.integers(1, min(E, 10) + 1))
        T = int(rng.integers(0, 40))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
            np.zeros((0, k), np.int32)
        if rng.random() < 0.3 and T:
            idx = np.minimum(idx, 2)  # heavy reuse (duplicates within a token are not
            # produced by routing but bucketing must still be a stable sort)
        b = oracle.bucket_routes(idx, E)
        flat = idx.reshape(-1)
        R = flat.size
        assert b["expert_count"].sum() == R
        assert np.array_equal(b["expert_count"], np.bincount(flat, minlength=E))
        assert np.array_equal(b["expert_offset"], np.concatenate([[0], np.cumsum(b["expert_count"])]))
        act = np.flatnonzero(b["expert_count"])
        assert int(b["n_active"]) == act.size
        assert np.array_equal(b["active_experts"][: act.size], act)
        assert np.all(b["active_experts"][act.size:] == -1)
        order = np.lexsort((np.arange(R), flat))
        assert np.array_equal(b["route_src"], order)
        assert np.array_equal(b["route_pos"][b["route_src"]], np.arange(R))


# ---------------------------------------------------------------- FFN (P5, P8-P14)

def check_ffn_golden():
    for case in load_golden("ffn_hand_worked.json")["cases"]:
        bank = bank_from_case(case)
        x = x_from_case(case)
        logits = np.array(case["logits"], dtype=np.float32)
        idx, w = oracle.route_topk(logits, None, case["k"])
        assert idx.tolist() == case["idx"]
        y = oracle.moe_output(x, bank, idx, w)
        exp_even, exp_odd = _ev(case["y"]["even"]), _ev(case["y"]["odd"])
        assert np.allclose(y[:, 0::2], exp_even, rtol=1e-14, atol=0), (case["name"], y[0, :4])
        assert np.allclose(y[:, 1::2], exp_odd, rtol=1e-14, atol=0), (case["name"], y[0, :4])


def check_single_expert_is_dense(seed: int = 3):
    """k = 1: weight 1 and y equals the dense SwiGLU FFN of the chosen expert."""
    rng = np.random.default_rng(seed)
    E, H, I, T = 3, 32, 48, 3
    bank, dense = random_grid_bank(rng, E, H, I)
    x = rng.integers(0, 1 << 16, size=(T, H)).astype(np.uint16)
    x = (x & 0x807F) | 0x3F00   # finite bf16 values in [-2, 2)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, None, 1)
    assert np.all(w == 1.0)
    y = oracle.moe_output(x, bank, idx, w)
    for t in range(T):
        ref = dense_swiglu_exact(bf16_values(x[t]), *dense[int(idx[t, 0])])
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), t


def check_mixture_matches_dense(seed: int = 4):
    """k > 1: y_t equals sum_j w_j * dense_FFN_{e_j}(x_t) (exact dots)."""
    rng = np.random.default_rng(seed)
    E, H, I, T, k = 6, 32, 32, 4, 3
    bank, dense = random_grid_bank(rng, E, H, I)
    x = ((rng.integers(0, 1 << 16, size=(T, H)).astype(np.uint16) & 0x807F) | 0x3F00).astype(np.uint16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, None, k)
    y = oracle.moe_output(x, bank, idx, w)
    for t in range(T):
        parts = [dense_swiglu_exact(bf16_values(x[t]), *dense[int(e)]) for e in idx[t]]
        ref = np.array([math.fsum(w[t, j] * parts[j][h] for j in range(k)) for h in range(H)])
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), t


def check_zero_input():
    """x = 0: logits +0, slots [0..k-1], weights 1/k, output exactly 0."""
    from moe_inputs import router_logits
    rng = np.random.default_rng(6)
    E, H, I, T, k = 8, 32, 32, 3, 3
    bank, _ = random_grid_bank(rng, E, H, I)
    x = np.zeros((T, H), np.uint16)
    logits = router_logits(x, rng.standard_normal((E, H)).astype(np.float32))
    assert np.all(logits == 0)
    idx, w = oracle.route_topk(logits, None, k)
    assert np.array_equal(idx, np.tile(np.arange(k), (T, 1)))
    assert np.all(w == 1.0 / k)
    y = oracle.moe_output(x, bank, idx, w)
    assert np.all(y == 0)


def check_all_equal_experts():
    """A bias sends every token to the same k experts."""
    rng = np.random.default_rng(7)
    E, H, I, T, k = 8, 32, 32, 5, 3
    bank, dense = random_grid_bank(rng, E, H, I)
    chosen = [2, 5, 6]
    bias = np.zeros(E, np.float32)
    bias[chosen] = 100.0
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, bias, k)
    assert all(sorted(r) == chosen for r in idx.tolist())
    b = oracle.bucket_routes(idx, E)
    assert int(b["n_active"]) == k
    assert b["expert_count"][chosen].tolist() == [T] * k
    x = ((rng.integers(0, 1 << 16, size=(T, H)).astype(np.uint16) & 0x807F) | 0x3F00).astype(np.uint16)
    y = oracle.moe_output(x, bank, idx, w)
    for t in range(T):
        parts = [dense_swiglu_exact(bf16_values(x[t]), *dense[int(e)]) for e in idx[t]]
        ref = sum(w[t, j] * parts[j] for j in range(k))
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def check_all_disjoint_experts():
    """T*k <= E and token t scores experts t*k..t*k+k-1 highest: all counts 1,
    bucket order is the identity."""
    T, k, E = 3, 2, 8
    logits = np.zeros((T, E), np.float32)
    for t in range(T):
        for j in range(k):
            logits[t, t * k + j] = 10.0 - j
    idx, _ = oracle.route_topk(logits, None, k)
    assert idx.tolist() == [[t * k + j for j in range(k)] for t in range(T)]
    b = oracle.bucket_routes(idx, E)
    assert b["expert_count"].tolist() == [1] * (T * k) + [0] * (E - T * k)
    assert np.array_equal(b["route_src"], np.arange(T * k))
    assert np.array_equal(b["route_pos"], np.arange(T * k))


def check_symmetries():
    rng = np.random.default_rng(8)
    E, H, I, T, k = 6, 32, 32, 4, 2
    bank, _ = random_grid_bank(rng, E, H, I)
    x = ((rng.integers(0, 1 << 16, size=(T, H)).astype(np.uint16) & 0x807F) | 0x3F00).astype(np.uint16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, None, k)
    y = oracle.moe_output(x, bank, idx, w)
    # run-to-run identical
    assert np.array_equal(y, oracle.moe_output(x, bank, idx, w))
    # doubling every down global scale doubles y exactly
    from types import SimpleNamespace
    b2 = SimpleNamespace(**vars(bank))
    b2.g_scale = bank.g_scale.copy()
    b2.g_scale[:, 2] *= 2
    assert np.array_equal(oracle.moe_output(x, b2, idx, w), 2 * y)
    # permuting tokens permutes rows
    perm = rng.permutation(T)
    idx_p, w_p = oracle.route_topk(logits[perm], None, k)
    assert np.array_equal(oracle.moe_output(x[perm], bank, idx_p, w_p), y[perm])
    # duplicated tokens give identical rows
    xd = np.concatenate([x, x[:1]])
    ld = np.concatenate([logits, logits[:1]])
    idx_d, w_d = oracle.route_topk(ld, None, k)
    yd = oracle.moe_output(xd, bank, idx_d, w_d)
    assert np.array_equal(yd[-1], yd[0])


# ---------------------------------------------------------------- router projection

def check_router_integers_exact():
    """Integer activations (exact in bf16) and integer weights: every sum is an
    integer below 2^24, so the logits are those integers exactly; T, E and H
    all differ, so a transposed operand cannot pass."""
    rng = np.random.default_rng(20)
    T, E, H = 3, 5, 64
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-100, 101, size=(E, H))
    x_bits = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_values(x_bits), xi.astype(np.float64))
    got = oracle.router_logits(x_bits, wi.astype(np.float32))
    want = np.array([[int(np.dot(xi[t], wi[e])) for e in range(E)] for t in range(T)], dtype=np.float32)
    assert got.dtype == np.float32 and got.shape == (T, E)
    assert np.array_equal(got, want)


def _round_f32_exact(q):
    """Round a Fraction to the nearest float32, ties to even mantissa."""
    from fractions import Fraction
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda f: (abs(Fraction(float(f)) - q), int(np.float32(f).view(np.uint32)) & 1))


def check_router_exact_rounding():
    """Random bf16 activations and fp32 weights: each logit is the float32
    nearest the exact rational sum (fractions.Fraction), i.e. one rounding."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    for _ in range(6):
        T, E, H = 3, 4, 48
        xf = rng.standard_normal((T, H)).astype(np.float32)
        x_bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
        w = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
        got = oracle.router_logits(x_bits, w)
        xv = bf16_values(x_bits)
        for t in range(T):
            for e in range(E):
                q = sum((Fraction(float(xv[t, h])) * Fraction(float(w[e, h])) for h in range(H)), Fraction(0))
                assert got[t, e] == _round_f32_exact(q), (t, e, got[t, e], float(q))


ALL_PINS = [
    check_e2m1, check_e4m3, check_products_exact_in_bf16, check_dequant_layout,
    check_routing_golden, check_topk_bruteforce, check_weight_invariants,
    check_buckets, check_ffn_golden, check_single_expert_is_dense,
    check_mixture_matches_dense, check_zero_input, check_all_equal_experts,
    check_all_disjoint_experts, check_symmetries,
    check_router_integers_exact, check_router_exact_rounding,
]
