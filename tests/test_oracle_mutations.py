"""Planted mistakes in the oracle must be caught by its pins.

A negative test must break the real rule, not a no-op: each mutation below
changes one rule the oracle follows (tie-break, renormalisation, nibble order,
SiLU, bias, stable bucket order, slot order of the weights) and asserts that
at least one pin fails.  The mistakes are planted on the CPU, in the oracle,
through monkeypatching; the oracle's source is untouched.
"""

import numpy as np
import pytest

import oracle
import oracle.buckets
import oracle.ffn
import oracle.formats
import oracle.route
import oracle.router
import pins


def _expect_failure(checks):
    failed = []
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "no pin caught the planted mistake"
    return failed


def test_flipped_tie_break(monkeypatch):
    monkeypatch.setattr(oracle.route, "_selection_key", lambda v, e: (-v, -e))
    _expect_failure([pins.check_routing_golden, pins.check_topk_bruteforce])


def test_no_renormalisation(monkeypatch):
    monkeypatch.setattr(oracle.route, "_renormalise", lambda p: p)
    _expect_failure([pins.check_weight_invariants, pins.check_routing_golden])


def test_swapped_nibbles(monkeypatch):
    def swapped(packed):
        packed = np.asarray(packed, dtype=np.uint8)
        out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
        out[..., 0::2] = packed >> 4
        out[..., 1::2] = packed & 0xF
        return out
    monkeypatch.setattr(oracle.formats, "unpack_nibbles", swapped)
    _expect_failure([pins.check_ffn_golden, pins.check_dequant_layout])


def test_wrong_silu_sign(monkeypatch):
    import numpy as _np
    monkeypatch.setattr(oracle.ffn, "silu", lambda v: v / (1.0 + _np.exp(v)))
    _expect_failure([pins.check_ffn_golden, pins.check_single_expert_is_dense])


def test_bias_ignored(monkeypatch):
    orig = oracle.route.biased_scores
    monkeypatch.setattr(oracle.route, "biased_scores", lambda logits, bias: orig(logits, None))
    _expect_failure([pins.check_routing_golden, pins.check_all_equal_experts])


def test_unstable_bucket_order(monkeypatch):
    orig = oracle.buckets.bucket_routes

    def reversed_within_expert(topk_idx, E):
        b = orig(topk_idx, E)
        flat = np.asarray(topk_idx).reshape(-1)
        src = np.array(sorted(range(flat.size), key=lambda r: (flat[r], -r)), dtype=np.int32)
        b["route_src"] = src
        b["route_pos"][src] = np.arange(flat.size, dtype=np.int32)
        return b
    monkeypatch.setattr(oracle, "bucket_routes", reversed_within_expert)
    _expect_failure([pins.check_buckets])


def test_weights_in_wrong_slots(monkeypatch):
    orig = oracle.route.renormalised_weights
    monkeypatch.setattr(oracle.route, "renormalised_weights",
                        lambda z, sel: orig(z, sel)[::-1].copy())
    _expect_failure([pins.check_routing_golden, pins.check_weight_invariants,
                     pins.check_mixture_matches_dense])


def test_wrong_scale_block(monkeypatch):
    def shifted(packed, scales, g):
        codes = oracle.formats.unpack_nibbles(packed)
        vals = oracle.formats.E2M1_VALUES[codes]
        s = oracle.formats._E4M3[np.asarray(scales, dtype=np.uint8)]
        return vals * np.repeat(s, 32, axis=1)[:, : codes.shape[1]] * float(g)
    monkeypatch.setattr(oracle.formats, "dequant_nvfp4", shifted)
    monkeypatch.setattr(oracle.ffn, "dequant_nvfp4", shifted)
    _expect_failure([pins.check_ffn_golden, pins.check_dequant_layout,
                     pins.check_single_expert_is_dense])


def test_router_summed_in_fp32(monkeypatch):
    def fp32_sum(x_bf16, w_router):
        x = oracle.formats.bf16_bits_to_f64(np.asarray(x_bf16, np.uint16)).astype(np.float32)
        w = np.asarray(w_router, np.float32)
        out = np.zeros((x.shape[0], w.shape[0]), np.float32)
        for h in range(x.shape[1]):                     # one fp32 rounding per term
            out = (out + np.outer(x[:, h], w[:, h])).astype(np.float32)
        return out
    monkeypatch.setattr(oracle.router, "router_logits", fp32_sum)
    monkeypatch.setattr(oracle, "router_logits", fp32_sum)
    _expect_failure([pins.check_router_exact_rounding])


def test_router_transposed(monkeypatch):
    def transposed(x_bf16, w_router):
        x = oracle.formats.bf16_bits_to_f64(np.asarray(x_bf16, np.uint16))
        w = np.asarray(w_router, np.float32).astype(np.float64)
        return (x @ w.reshape(w.shape[1], w.shape[0])).astype(np.float32)
    monkeypatch.setattr(oracle.router, "router_logits", transposed)
    monkeypatch.setattr(oracle, "router_logits", transposed)
    _expect_failure([pins.check_router_integers_exact])
