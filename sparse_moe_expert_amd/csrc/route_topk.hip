// moe_route_topk: softmax top-k routing with renormalised gate weights.
//
// Selection follows the fused MoE routing kernel's rule (page "How I forked
// vLLM and made Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section
// "5. Hand-written kernels", paragraph "Fused MoE routing"): repeated arg-max
// over the scores with the lowest expert id winning ties, lanes holding
// contiguous experts read with vector loads.  The SM70 note's router section
// states the same tie rule for its repeated-maxima selection (page
// "Persistent execution for Flash-Next GGUF on SM70", section "Router:
// selection and expert-task production").
//
// Mapping (gfx950): one 64-lane wavefront per token, four tokens per
// 256-thread workgroup.  Lane l holds experts [l*V, l*V+V) as 64-bit keys
//   key = ordered(z) << 32 | (0xFFFFFFFF - e)
// where ordered() maps fp32 to an unsigned integer with the same order
// (-0.0 first canonicalised to +0.0).  The maximum key is the largest z with
// the lowest id.  Each of the k rounds takes a per-lane maximum and a
// butterfly maximum across the wave; the owner lane then retires the winner.
#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t ordered_bits(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0;                 // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int V>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                           // whole wavefront leaves together
  const float* row = logits + (size_t)t * E;
  const int e0 = lane * V;

  float zv[V];
  const bool full = (V % 4 == 0) && (E % 4 == 0) && (e0 + V <= E);
  if (full) {                                   // 16-byte vector loads
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const float4 l4 = *reinterpret_cast<const float4*>(row + e0 + i);
      zv[i] = l4.x; zv[i + 1] = l4.y; zv[i + 2] = l4.z; zv[i + 3] = l4.w;
      if (bias) {
        const float4 b4 = *reinterpret_cast<const float4*>(bias + e0 + i);
        zv[i] += b4.x; zv[i + 1] += b4.y; zv[i + 2] += b4.z; zv[i + 3] += b4.w;  // fp32 adds, RNE
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = e0 + i;
      zv[i] = 0.0f;
      if (e < E) zv[i] = bias ? row[e] + bias[e] : row[e];
    }
  }
  uint64_t key[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = e0 + i;
    key[i] = (e < E) ? (((uint64_t)ordered_bits(zv[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e))
                     : 0;                       // 0 sorts below every real key
  }

  // Selected scores live in lane j (slot j) after the loop.
  float my_z = 0.0f;
  int my_e = 0;
  float z0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < V; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float z = from_ordered((uint32_t)(best >> 32));
    if (j == 0) z0 = z;
    if (lane == j) { my_z = z; my_e = e; }
    // retire the winner in its owner lane
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (e0 + i == e) key[i] = 0;
  }

  // Renormalised softmax over the chosen set: w_j = exp(z_j - z_0) / sum.
  // The sum runs in slot order j = 0..k-1 on every lane (fixed order).
  const float p = (lane < k) ? __builtin_expf(my_z - z0) : 0.0f;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s += __shfl(p, j, kWave);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = p / s;
  }
}

}  // namespace

}  // namespace moe

extern "C" moe_status moe_route_topk(const float* logits, const float* bias, int T, int E, int k,
                                     int32_t* topk_idx, float* topk_w, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL_POINTER;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w) || (bias && !aligned16(bias)))
    return MOE_ERR_MISALIGNED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((T + 3) / 4), block(256);
  const int V = (E + kWave - 1) / kWave;
  if (V <= 1) route_topk_kernel<1><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 2) route_topk_kernel<2><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 4) route_topk_kernel<4><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 8) route_topk_kernel<8><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else route_topk_kernel<16><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  return launch_status();
}
