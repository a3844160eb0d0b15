"""The five routed-MoE workloads (shapes, routing distributions, seeds).

Shapes: the Flash-Next MoE has 512 experts with top-10 routing and NVFP4
expert weights (page "How I forked vLLM and made Qwen3.8-Flash-Next decode
1.6x faster on one GPU", section "The model and the constraint").  T=4 is one
decode step verifying 3 MTP drafts (TokenSpeed Flash-Next blog, "Serving
benchmarks": 3 draft steps, 4 verification tokens).  The expert sizes H=2048,
I=512 and the three larger token counts (32, 256, 4096) define the batched,
skewed and prefill regimes.

Routing distributions (readings where the description is brief):
  * "none"   - logits only: x ~ N(0,1) projected by W_r ~ N(0, 1/H).
  * "normal" - plus a per-expert bias drawn N(0, 0.5), 0.5 being the variance
               (the same convention as N(0, 1/H) for W_r).
  * "zipf"   - plus bias[perm[r-1]] = -s * ln(r) for rank r = 1..E, i.e. the log
               of unnormalised Zipf(s) weights over a seeded expert permutation.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts
    k: int          # experts per token
    bias: str       # "none" | "normal" | "zipf"
    bias_param: float = 0.0   # variance for "normal", exponent s for "zipf"
    seed: int = 0
    description: str = ""

    @property
    def routes(self) -> int:
        return self.T * self.k

    def expert_bytes(self) -> int:
        """NVFP4 bytes of one expert: codes + e4m3 block scales of 3 matrices."""
        per_matrix = self.H * self.I // 2 + self.H * self.I // 16
        return 3 * per_matrix


CONFIGS = {
    "tiny": WorkloadConfig(
        "tiny", T=4, H=256, I=128, E=8, k=2, bias="none",
        description="Tiny MoE FFN, T=4 H=256 I=128 E=8 top-2"),
    "decode_t4": WorkloadConfig(
        "decode_t4", T=4, H=2048, I=512, E=512, k=10, bias="none",
        description="Decode verify step, B=1 with 3 MTP drafts: T=4 E=512 top-10"),
    "verify_t32": WorkloadConfig(
        "verify_t32", T=32, H=2048, I=512, E=512, k=10, bias="normal", bias_param=0.5,
        description="Batched verify, 8 requests x 4 tokens, per-expert bias N(0,0.5)"),
    "decode_t256_zipf": WorkloadConfig(
        "decode_t256_zipf", T=256, H=2048, I=512, E=512, k=10, bias="zipf", bias_param=1.1,
        description="Large decode batch T=256, Zipf(1.1)-skewed routing"),
    "prefill_t4096": WorkloadConfig(
        "prefill_t4096", T=4096, H=2048, I=512, E=512, k=10, bias="none",
        description="Prefill chunk T=4096, uniform routing"),
}

# The Flash-Next expert as the pages size it, beside the five workloads:
# hidden 2560 and expert intermediate 640, i.e. 3 * (2560*640/2 + 2560*640/16)
# = 2.637 MiB of NVFP4 per expert (page "Qwen3.8 Flash Next on LiL/vLLM: why
# the MTP decode step is host-bound, and what LMCache does and does not do to
# it", section "11.13 Where the decode step's time actually goes"), K = 2560
# with 512 experts and N = 160 per rank of four (page "Persistent execution
# for Flash-Next GGUF on SM70", section "Primary sources and transferable
# mechanisms", paragraph "MonoMoE").  Their rows hold 80 and 20 16-byte
# chunks, which are not powers of two.
EXTRA_CONFIGS = {
    "flashnext_t4": WorkloadConfig(
        "flashnext_t4", T=4, H=2560, I=640, E=512, k=10, bias="none",
        description="Decode verify step at the Flash-Next expert shape H=2560 I=640, T=4 E=512 top-10"),
    "flashnext_t256": WorkloadConfig(
        "flashnext_t256", T=256, H=2560, I=640, E=512, k=10, bias="none",
        description="256-token batch at the Flash-Next expert shape H=2560 I=640, E=512 top-10"),
}

# Stable order used by tests and reports.
CONFIG_ORDER = ["tiny", "decode_t4", "verify_t32", "decode_t256_zipf", "prefill_t4096"]


def get_config(name: str) -> WorkloadConfig:
    try:
        return CONFIGS[name] if name in CONFIGS else EXTRA_CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_ORDER}") from None
