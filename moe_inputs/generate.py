"""Seeded generation of routed-MoE inputs.

Random streams (numpy PCG64 seeded with SeedSequence([seed, stream])), so that
every workload at the Flash-Next shape shares one model (router and expert
weights) while the activations change with the token count:
  stream 0: activations x ~ N(0, 1), drawn in fp64 -> fp32 -> bf16 (RNE each step)
  stream 1: expert weights; expert e draws from SeedSequence([seed, 1, e]):
            W_gate [I,H], W_up [I,H], W_down [H,I] ~ N(0, 1/fan_in) (fan_in H, H, I), fp32
  stream 2: router weights W_r [E,H] ~ N(0, 1/H), fp32
  stream 3: routing bias ("normal": N(0, var) per expert; "zipf": a permutation)

Router logits are the prerequisite projection that sits outside the routed
step (the MonoMoE host wrapper receives precomputed router logits; the SM70
design note keeps the router GEMV as an explicit prerequisite - page
"Persistent execution for Flash-Next GGUF on SM70", sections "MonoMoE" and
"First implementation boundary").  They are computed here once, in fp64 from
the bf16 activations and fp32 router weights, and rounded once to fp32, so
that the GPU path and the oracle consume the same logits tensor.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import WorkloadConfig, get_config
from .nvfp4_encode import encode_nvfp4

STREAM_X, STREAM_EXPERTS, STREAM_ROUTER, STREAM_BIAS = 0, 1, 2, 3


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16 (finite inputs)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _bf16_bits_as_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x_bf16: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """fp32(x @ W_r^T) computed in fp64 and rounded once."""
    return (_bf16_bits_as_f64(x_bf16) @ w_router.astype(np.float64).T).astype(np.float32)


@dataclass
class ExpertBank:
    """NVFP4 expert weights of E experts (row-major, rows along the output)."""
    w_gate: np.ndarray   # uint8 [E, I, H/2]
    s_gate: np.ndarray   # uint8 [E, I, H/16]
    w_up: np.ndarray     # uint8 [E, I, H/2]
    s_up: np.ndarray     # uint8 [E, I, H/16]
    w_down: np.ndarray   # uint8 [E, H, I/2]
    s_down: np.ndarray   # uint8 [E, H, I/16]
    g_scale: np.ndarray  # float32 [E, 3] (gate, up, down)


_BANK_CACHE: dict = {}


def _expert_tensors(seed: int, e: int, H: int, I: int):
    """Draw and encode expert e from its own stream SeedSequence([seed, 1, e])."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, STREAM_EXPERTS, e]))
    z = rng.standard_normal((3, I * H), dtype=np.float32)
    wg = (z[0] * np.float32(1.0 / np.sqrt(H))).reshape(1, I, H)
    wu = (z[1] * np.float32(1.0 / np.sqrt(H))).reshape(1, I, H)
    wd = (z[2] * np.float32(1.0 / np.sqrt(I))).reshape(1, H, I)
    return encode_nvfp4(wg), encode_nvfp4(wu), encode_nvfp4(wd)


def make_expert_bank(E: int, H: int, I: int, seed: int = 0, threads: Optional[int] = None) -> ExpertBank:
    """Draw and NVFP4-encode E experts (cached per (E, H, I, seed)).

    Expert e depends only on (seed, e), so experts are generated concurrently
    on a thread pool (numpy releases the GIL inside bulk draws and ufuncs).
    """
    key = (E, H, I, seed)
    if key in _BANK_CACHE:
        return _BANK_CACHE[key]
    bank = ExpertBank(
        w_gate=np.empty((E, I, H // 2), np.uint8), s_gate=np.empty((E, I, H // 16), np.uint8),
        w_up=np.empty((E, I, H // 2), np.uint8), s_up=np.empty((E, I, H // 16), np.uint8),
        w_down=np.empty((E, H, I // 2), np.uint8), s_down=np.empty((E, H, I // 16), np.uint8),
        g_scale=np.empty((E, 3), np.float32))

    def fill(e):
        (cg, sg, gg), (cu, su, gu), (cd, sd, gd) = _expert_tensors(seed, e, H, I)
        bank.w_gate[e], bank.s_gate[e], bank.g_scale[e, 0] = cg[0], sg[0], gg[0]
        bank.w_up[e], bank.s_up[e], bank.g_scale[e, 1] = cu[0], su[0], gu[0]
        bank.w_down[e], bank.s_down[e], bank.g_scale[e, 2] = cd[0], sd[0], gd[0]

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or E * H * I < (1 << 22):
        for e in range(E):
            fill(e)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(E)))
    _BANK_CACHE[key] = bank
    return bank


@dataclass
class Workload:
    cfg: WorkloadConfig
    x: np.ndarray                 # uint16 [T, H] bf16 bits
    w_router: np.ndarray          # float32 [E, H]
    logits: np.ndarray            # float32 [T, E]
    bias: Optional[np.ndarray]    # float32 [E] or None
    bank: Optional[ExpertBank]    # None when built with with_bank=False

    # convenience accessors
    @property
    def T(self): return self.cfg.T
    @property
    def H(self): return self.cfg.H
    @property
    def I(self): return self.cfg.I
    @property
    def E(self): return self.cfg.E
    @property
    def k(self): return self.cfg.k


def make_bias(cfg: WorkloadConfig, seed: int) -> Optional[np.ndarray]:
    if cfg.bias == "none":
        return None
    rng = _rng(seed, STREAM_BIAS)
    if cfg.bias == "normal":
        return (rng.standard_normal(cfg.E) * np.sqrt(cfg.bias_param)).astype(np.float32)
    if cfg.bias == "zipf":
        perm = rng.permutation(cfg.E)
        b = np.empty(cfg.E, np.float64)
        b[perm] = -cfg.bias_param * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))
        return b.astype(np.float32)
    raise ValueError(f"unknown bias kind {cfg.bias!r}")


def make_workload(cfg, seed: Optional[int] = None, x_seed: Optional[int] = None,
                  T: Optional[int] = None, with_bank: bool = True) -> Workload:
    """Build a workload.  `seed` fixes the model (router, bias, experts),
    `x_seed` the activations (defaults to `seed`); `T` overrides the token count."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    if T is not None and T != cfg.T:
        from dataclasses import replace
        cfg = replace(cfg, T=T)
    seed = cfg.seed if seed is None else seed
    x_seed = seed if x_seed is None else x_seed
    x = f64_to_bf16_bits(_rng(x_seed, STREAM_X).standard_normal((cfg.T, cfg.H)))
    w_router = (_rng(seed, STREAM_ROUTER).standard_normal((cfg.E, cfg.H))
                * np.sqrt(1.0 / cfg.H)).astype(np.float32)
    logits = router_logits(x, w_router)
    bias = make_bias(cfg, seed)
    bank = make_expert_bank(cfg.E, cfg.H, cfg.I, seed) if with_bank else None
    return Workload(cfg=cfg, x=x, w_router=w_router, logits=logits, bias=bias, bank=bank)
