// Top-k selection of one token per wavefront and wavefront scans (gfx950).
//
// Selection: lane l holds experts [l*V, l*V+V) with keys ordered(z), an
// unsigned integer with the same order as the fp32 score (-0.0 first
// canonicalised to +0.0); absent experts hold 0, below every real key.  Each
// of the k rounds takes the wave maximum of the lanes' leading keys, then the
// lowest lane holding it (ballot).
#pragma once

#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t ordered_bits(float z) {
  uint32_t u = __float_as_uint(z);
  u = (u == 0x80000000u) ? 0u : u;             // -0.0 == +0.0
  // negative: all bits flipped; otherwise the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// DPP with a row mask: rows outside `ROW_MASK` get 0 (the identity of the
// unsigned max and of the sum below).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_rows_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Maximum over the wavefront (wave-uniform result).  DPP steps reduce each
// 16-lane row; row broadcasts of lanes 15 and 31 then carry the row maxima
// up to lane 63, which is read once.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));              // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));              // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124>(v));             // row_ror:4
  v = max(v, dpp_u32<0x128>(v));             // row_ror:8: every lane holds its row's max
  v = max(v, dpp_rows_u32<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_rows_u32<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the wavefront in a fixed order (wave-uniform result): rows first,
// then (row3 + row2) + (row1 + row0) in lane 63.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [](float a, uint32_t b) { return a + __builtin_bit_cast(float, b); };
  v = add(v, dpp_u32<0xB1>(__builtin_bit_cast(uint32_t, v)));
  v = add(v, dpp_u32<0x4E>(__builtin_bit_cast(uint32_t, v)));
  v = add(v, dpp_u32<0x124>(__builtin_bit_cast(uint32_t, v)));
  v = add(v, dpp_u32<0x128>(__builtin_bit_cast(uint32_t, v)));
  v = add(v, dpp_rows_u32<0x142, 0xA>(__builtin_bit_cast(uint32_t, v)));
  v = add(v, dpp_rows_u32<0x143, 0xC>(__builtin_bit_cast(uint32_t, v)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

constexpr uint32_t kIdMask = 1023;             // expert ids < 1024

// Top-k of one token's row: idx/weights of slot j end up in lane j.
//
// Each lane first sorts its V (score, id) pairs as 64-bit keys - ordered(z)
// in the high word, 1023 - id in the low word, so one unsigned comparison
// orders by score descending and id ascending - with a bitonic network.  A
// round then only needs the wave maximum of the lanes' leading scores, the
// lowest lane holding it (lanes own ascending id ranges, so that is the
// lowest id among equal scores) and a one-step shift of that lane's list:
// no per-round rescan and no divergent branch.
//
// KC > 0 fixes k = KC at compile time: the rounds are then unrolled into one
// straight-line block, so the shift of one round's winning list can fill the
// wait states of the next round's reduction (k is then ignored).
// Lane l's V (score, id) keys of one token's row, sorted descending - see
// select_token.
template <int V>
__device__ __forceinline__ void sorted_keys(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                            int lane, uint64_t (&K)[V]) {
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
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool ok = e0 + i < E;
    const uint32_t hi = ok ? ordered_bits(zv[i]) : 0u, lo = ok ? kIdMask - (uint32_t)(e0 + i) : 0u;
    K[i] = ((uint64_t)hi << 32) | lo;
  }
#pragma unroll
  for (int size = 2; size <= V; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;      // the last stage (size == V) is all descending
          const uint64_t a = K[i], b = K[j];
          // one comparison per exchange: an opaque all-ones/zero mask and
          // bitwise selects (plain selects become separate max and min)
          uint32_t m = (desc ? (b > a) : (a > b)) ? 0xFFFFFFFFu : 0u;
          asm("" : "+v"(m));
          const uint64_t m64 = ((uint64_t)m << 32) | m;
          K[i] = (b & m64) | (a & ~m64);
          K[j] = (a & m64) | (b & ~m64);
        }
      }
    }
  }
}

// One round: the wave maximum of the lanes' leading keys (*best, wave
// uniform) and its expert id (returned); the winning lane drops its leading
// key.  The all-ones/zero mask is made opaque so the compiler keeps V
// bitwise selects (v_bfi) instead of rewriting the shift as a lane-dependent
// index into K, which it lowers to V*V selects.
template <int V>
__device__ __forceinline__ int select_round(uint64_t (&K)[V], int lane, uint32_t* best) {
  const uint32_t lead = (uint32_t)(K[0] >> 32);
  const uint32_t wbest = wave_max_u32(lead);
  const int wl = __builtin_ctzll(__ballot(lead == wbest));
  const uint32_t low = __builtin_amdgcn_readlane((uint32_t)K[0], wl);
  *best = wbest;
  uint32_t m = lane == wl ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  const uint64_t m64 = ((uint64_t)m << 32) | m;
#pragma unroll
  for (int i = 0; i + 1 < V; ++i) K[i] = (K[i + 1] & m64) | (K[i] & ~m64);
  K[V - 1] &= ~m64;
  return (int)(kIdMask - (low & kIdMask));
}

// Top-k of one token's row: idx/weights of slot j end up in lane j.
//
// Each lane first sorts its V (score, id) pairs as 64-bit keys - ordered(z)
// in the high word, 1023 - id in the low word, so one unsigned comparison
// orders by score descending and id ascending - with a bitonic network.  A
// round then only needs the wave maximum of the lanes' leading scores, the
// lowest lane holding it (lanes own ascending id ranges, so that is the
// lowest id among equal scores) and a one-step shift of that lane's list:
// no per-round rescan and no divergent branch.
//
// KC > 0 fixes k = KC at compile time: the rounds are then unrolled into one
// straight-line block, so the shift of one round's winning list can fill the
// wait states of the next round's reduction (k is then ignored).
template <int V, int KC = 0>
__device__ __forceinline__ void select_token(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                             int k, int lane, int& my_e, float& my_w) {
  uint64_t K[V];
  sorted_keys<V>(row, bias, E, lane, K);
  uint32_t my_key = 0, key0 = 0;
  my_e = 0;
  auto round = [&](int j) {
    uint32_t wbest;
    const int e_sel = select_round<V>(K, lane, &wbest);
    if (j == 0) key0 = wbest;
    if (lane == j) { my_key = wbest; my_e = e_sel; }
  };
  if constexpr (KC > 0) {
#pragma unroll
    for (int j = 0; j < KC; ++j) round(j);
  } else {
    for (int j = 0; j < k; ++j) round(j);
  }
  // Renormalised softmax over the chosen set: w_j = exp(z_j - z_0) / sum.
  const float z0 = from_ordered(key0);
  const int kk = KC > 0 ? KC : k;
  const float pj = (lane < kk) ? __builtin_expf(from_ordered(my_key) - z0) : 0.0f;
  my_w = pj / wave_sum_f32(pj);
}

// The expert of slot j alone (wave uniform): the rounds of select_token up
// to round j, so slot 0 costs one round and slot k - 1 all k of them.  With
// KC > 0 the rounds are unrolled up to KC and left early.
template <int V, int KC = 0>
__device__ __forceinline__ int select_slot(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                           int j, int lane) {
  uint64_t K[V];
  sorted_keys<V>(row, bias, E, lane, K);
  uint32_t wbest;
  int e = 0;
  if constexpr (KC > 0) {
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      e = select_round<V>(K, lane, &wbest);
      if (r == j) break;
    }
  } else {
    for (int r = 0; r <= j; ++r) e = select_round<V>(K, lane, &wbest);
  }
  return e;
}

// Inclusive scan across a 64-lane wavefront with DPP: shifts of 1, 2, 4, 8
// inside each 16-lane row (lanes without a source add 0), then row broadcasts
// of lanes 15 and 31 into the rows above them.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_shift(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_shift<0x111, 0xF>(v);   // row_shr:1
  v += dpp_shift<0x112, 0xF>(v);   // row_shr:2
  v += dpp_shift<0x114, 0xF>(v);   // row_shr:4
  v += dpp_shift<0x118, 0xF>(v);   // row_shr:8
  v += dpp_shift<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_shift<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}


// Exclusive scan of one value per thread over a workgroup of WAVES
// wavefronts; also returns the total.  s_wt: WAVES ints of LDS.
template <int WAVES>
__device__ __forceinline__ int block_scan(int v, int* s_wt, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wt[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const int t = s_wt[w];
    base += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();
  return base + inc - v;
}

}  // namespace
}  // namespace moe
