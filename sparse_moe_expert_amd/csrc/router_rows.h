// The router projection's row body for small batches, shared by
// moe_router_logits and the fused projection + routing kernel (gfx950).
//
// logits[t, e] = fl32( sum_h x[t, h] * W_r[e, h] ): each bf16 x fp32 product
// is exact in fp64 (8 + 24 significant bits); the sum is accumulated in fp64
// in a fixed order and rounded once.
#pragma once

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kRtThreads = 256;
constexpr int kRtWaves = kRtThreads / kWave;
constexpr int kRtMaxH = 4096;          // the small-batch row body: two 8-value pieces per thread
constexpr int kRsMaxTokens = 64;       // batches up to this size: one 256-thread group per expert row

__device__ __forceinline__ double bf16_lo(uint32_t v) { return (double)__uint_as_float(v << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t v) { return (double)__uint_as_float(v & 0xFFFF0000u); }

// fp64 value moved by one DPP pattern (each 32-bit half with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wavefront in a fixed order; every lane gets the same bits.
// DPP steps sum each 16-lane row into all of its lanes; v_permlane16_swap and
// v_permlane32_swap (each applied to both halves) then add the rows pairwise:
// ((row0 + row1) + (row2 + row3)) - lanes of the other half form the same
// sums with the operands swapped, which fp64 addition does not distinguish.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f64<0x124>(v);   // row_ror:4
  v += dpp_f64<0x128>(v);   // row_ror:8
  auto swap_add = [](double a, bool rows32) {
    const uint64_t u = __builtin_bit_cast(uint64_t, a);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto l = rows32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                          : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = rows32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                          : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const double x0 = __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]);
    const double x1 = __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
    return x0 + x1;
  };
  v = swap_add(v, false);   // rows (0+1), (2+3) in every lane of their pair
  return swap_add(v, true); // (0+1) + (2+3)
}

// Small batches: one group of kRtThreads threads per expert row, so the row's
// loads and products spread over 256 lanes.  Thread i of the group holds the
// row's values h = 8(i + 256c) .. +8 as fp64 and reads the same 16 bytes of
// each token's activation row directly (cached: every group reads the same
// x), G (up to eight) tokens at a time - a batch of T <= 4 tokens takes the
// smallest G >= T, so no wavefront sum is formed for an absent token; the
// sums do not depend on G; wavefront sums go to LDS (s_part, the group's
// own) and are added in wave order.  Every thread of the workgroup calls it
// (it has workgroup barriers); a group whose row e lies past E computes
// nothing and stores nothing.
constexpr int kRsGroup = 8;

template <int NCH, int G = kRsGroup>
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x, const float* __restrict__ w, int T, int H,
                                           int E, float* __restrict__ logits, int e, int gtid,
                                           double (&s_part)[kRtWaves][kRsGroup]) {
  const int lane = gtid & (kWave - 1);
  const int wave = gtid >> 6;
  const bool row_ok = e < E;
  double wd[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int h0 = 8 * (gtid + kRtThreads * c);
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), b = a;
    if (row_ok && h0 < H) {
      a = *reinterpret_cast<const float4*>(w + (size_t)e * H + h0);
      b = *reinterpret_cast<const float4*>(w + (size_t)e * H + h0 + 4);
    }
    wd[c][0] = a.x; wd[c][1] = a.y; wd[c][2] = a.z; wd[c][3] = a.w;
    wd[c][4] = b.x; wd[c][5] = b.y; wd[c][6] = b.z; wd[c][7] = b.w;
  }
  static_assert(G >= 1 && G <= kRsGroup, "at most kRsGroup tokens per pass");
  for (int t0 = 0; t0 < T; t0 += G) {
    const int nt = min(G, T - t0);
    uint4 xv[G][NCH];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int h0 = 8 * (gtid + kRtThreads * c);
        xv[g][c] = make_uint4(0u, 0u, 0u, 0u);
        if (row_ok && g < nt && h0 < H) xv[g][c] = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + g) * H + h0);
      }
    double acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      double a = 0.0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t q[4] = {xv[g][c].x, xv[g][c].y, xv[g][c].z, xv[g][c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a = fma(wd[c][2 * i], bf16_lo(q[i]), a);
          a = fma(wd[c][2 * i + 1], bf16_hi(q[i]), a);
        }
      }
      acc[g] = wave_sum_f64(a);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) s_part[wave][g] = acc[g];
    }
    __syncthreads();
    if (row_ok && gtid < nt) {
      static_assert(kRtWaves == 4, "the wave partials are added pairwise");
      const double sum = (s_part[0][gtid] + s_part[1][gtid]) + (s_part[2][gtid] + s_part[3][gtid]);
      logits[(size_t)(t0 + gtid) * E + e] = (float)sum;
    }
    __syncthreads();                                   // s_part reused by the next group
  }
}

template <int NCH, int G>
__global__ __launch_bounds__(kRtThreads) void router_rows_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ w, int T, int H, int E,
                                                                 float* __restrict__ logits) {
  __shared__ double s_part[kRtWaves][kRsGroup];
  router_row<NCH, G>(x, w, T, H, E, logits, (int)blockIdx.x, (int)threadIdx.x, s_part);
}

}  // namespace
}  // namespace moe
