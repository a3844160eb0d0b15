"""Helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Acceptance (fixed before any kernel ran): expert ids and every bucket array
bit-exact; gate weights within 1e-6 absolute; the bf16 output within
max|y - y_ref| <= 2e-2 * rms(y_ref), rms over the compared outputs (exactly 0
when the reference is exactly 0).  That bound is the one for the five
workloads.  Small edge-case shapes outside them (a few dozen outputs per token)
can have max|y_ref| well above 5 * rms, where the bf16 rounding of the output
itself (relative 2^-8) already reaches the bound; their tests use
assert_output_rounded, which adds half a bf16 ulp of each reference value.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_moe_expert_amd as sme

DEV = torch.device("cuda:0")
W_TOL = 1e-6
Y_REL_TOL = 2e-2

_WEIGHTS = {}


def device_weights(bank) -> sme.ExpertWeights:
    key = id(bank)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = (bank, sme.expert_weights_from_numpy(bank, DEV))
    return _WEIGHTS[key][1]


_PACKED = {}


def device_packed(bank) -> torch.Tensor:
    """The bank's weights packed in MFMA tile order (moe_pack_weights), cached."""
    key = id(bank)
    if key not in _PACKED:
        _PACKED[key] = (bank, sme.pack_weights(device_weights(bank)))
    return _PACKED[key][1]


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_bits(x_u16: np.ndarray) -> torch.Tensor:
    return to_dev(np.ascontiguousarray(x_u16).view(np.int16))


def run_gpu(x_u16, logits, bias, bank, k, step: sme.MoeStep = None, path: str = "step"):
    """One step through the C ABI (moe_step, moe_step_packed, or the separate calls)."""
    T, H = x_u16.shape
    E = logits.shape[1]
    W = device_weights(bank)
    I = W.shape[2]
    st = step or sme.MoeStep(T, H, I, E, k, DEV, path=path)
    st.run(x_bits(x_u16), to_dev(logits.astype(np.float32)),
           None if bias is None else to_dev(bias.astype(np.float32)), W,
           packed=device_packed(bank) if st.path == "packed" else None)
    torch.cuda.synchronize()
    return collect(st)


def collect(st: sme.MoeStep, with_y: bool = True) -> dict:
    """Copy every output to the host (with_y False: routing outputs only,
    for calls that never wrote y)."""
    b = st.buckets
    out = {
        "idx": st.topk_idx.cpu().numpy(),
        "w": st.topk_w.cpu().numpy(),
        "expert_count": b.expert_count.cpu().numpy(),
        "expert_offset": b.expert_offset.cpu().numpy(),
        "active_experts": b.active_experts.cpu().numpy(),
        "n_active": b.n_active.cpu().numpy(),
        "route_src": b.route_src.cpu().numpy(),
        "route_pos": b.route_pos.cpu().numpy(),
    }
    if with_y:
        out["y"] = st.y.float().cpu().numpy().astype(np.float64)
        out["y_bits"] = st.y.view(torch.int16).cpu().numpy()
    return out


def assert_route(g: dict, idx_ref, w_ref):
    assert np.array_equal(g["idx"], idx_ref), np.argwhere(g["idx"] != idx_ref)[:5]
    err = np.max(np.abs(g["w"].astype(np.float64) - w_ref)) if w_ref.size else 0.0
    assert err <= W_TOL, err


def assert_buckets(g: dict, b_ref: dict):
    for name in ("expert_count", "expert_offset", "active_experts", "route_src", "route_pos"):
        assert np.array_equal(g[name], b_ref[name]), name
    assert int(g["n_active"][0]) == int(b_ref["n_active"])


def assert_output(y_gpu: np.ndarray, y_ref: np.ndarray, tag: str = ""):
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    if rms == 0.0:
        assert err == 0.0, f"{tag}: reference is exactly 0, max|y| = {err}"
    else:
        assert err <= Y_REL_TOL * rms, f"{tag}: max err {err:.3e} > {Y_REL_TOL} * rms {rms:.3e}"
    return err, rms


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits): the largest error of
    rounding an exact value to bf16."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, np.finfo(np.float32).tiny)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def assert_output_rounded(y_gpu: np.ndarray, y_ref: np.ndarray, tag: str = ""):
    """|y - y_ref| <= 2e-2 * rms(y_ref) + half a bf16 ulp of y_ref, elementwise."""
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    d = np.abs(y_gpu - y_ref)
    if rms == 0.0:
        assert float(d.max(initial=0.0)) == 0.0, f"{tag}: reference is exactly 0"
        return 0.0, 0.0
    bound = Y_REL_TOL * rms + bf16_half_ulp(y_ref)
    worst = int(np.argmax(d - bound))
    assert np.all(d <= bound), (f"{tag}: |err| {d.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} "
                                f"at y_ref {y_ref.flat[worst]:.3e} (rms {rms:.3e})")
    return float(d.max()), rms


def oracle_all(x_u16, logits, bias, bank, k, tokens=None):
    E = logits.shape[1]
    idx, w = oracle.route_topk(logits, bias, k)
    b = oracle.bucket_routes(idx, E)
    y = oracle.moe_output(x_u16, bank, idx, w, tokens=tokens)
    return idx, w, b, y
