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
// 256-thread workgroup.  Lane l holds experts [l*V, l*V+V) as 32-bit keys
// ordered(z), an unsigned integer with the same order as the fp32 score
// (-0.0 first canonicalised to +0.0); absent experts hold 0, below every
// real key.  Each of the k rounds takes the wave maximum of the lanes' best
// keys (DPP row steps, then the four row maxima as scalars), then the
// lowest lane holding that key (ballot): lanes own ascending id ranges, so
// that lane - and its first matching slot - has the lowest id among equal
// scores.  Only the winning lane recomputes its best key.
#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t ordered_bits(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0;                 // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the wavefront (wave-uniform result).  DPP steps reduce each
// 16-lane row; the four row results are then read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124>(v));   // row_ror:4
  v = max(v, dpp_u32<0x128>(v));   // row_ror:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum over the wavefront in a fixed order (wave-uniform result).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
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
  uint32_t key[V];
  uint32_t best = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    key[i] = (e0 + i < E) ? ordered_bits(zv[i]) : 0u;
    best = max(best, key[i]);
  }

  // slot j's score and id end up in lane j
  uint32_t my_key = 0;
  int my_e = 0;
  uint32_t key0 = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t wbest = wave_max_u32(best);
    const uint64_t holders = __ballot(best == wbest);
    const int wl = __builtin_ctzll(holders);    // lowest lane: lowest ids
    int pick = 0;
    if (lane == wl) {
      int first = V;
#pragma unroll
      for (int i = V - 1; i >= 0; --i)
        if (key[i] == wbest) first = i;
      pick = e0 + first;
      uint32_t nb = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (i == first) key[i] = 0;             // retire the winner
        nb = max(nb, key[i]);
      }
      best = nb;
    }
    const int e_sel = __builtin_amdgcn_readlane(pick, wl);
    if (j == 0) key0 = wbest;
    if (lane == j) { my_key = wbest; my_e = e_sel; }
  }

  // Renormalised softmax over the chosen set: w_j = exp(z_j - z_0) / sum.
  const float z0 = from_ordered(key0);
  const float p = (lane < k) ? __builtin_expf(from_ordered(my_key) - z0) : 0.0f;
  const float s = wave_sum_f32(p);
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
