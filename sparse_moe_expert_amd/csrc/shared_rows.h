// Row work of the dense BF16 shared expert (page "How I forked vLLM and made
// Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section "2. FP8 for the
// dense layers": shared experts stay BF16), one wavefront per weight row.
// The same functions serve the shared expert's own kernels and its rows
// riding along in the routed step's kernels, so both give the same bits.
//
// Gate/up row r: the wave holds rows r of W_gate and W_up (lane l, chunk c:
// values 8(l + 64c) .. +8, 16-byte loads), takes the tokens kSeTokens at a
// time (their x chunks issued together), multiplies bf16 pairs with
// v_dot2_f32_bf16 into fp32, sums the 64 lanes in a fixed butterfly order
// (wave_sum_xor) and
// writes h[t, r] = bf16(SiLU(g) * u).  Down rows c: the same with W_down's
// rows and h, writing y[t, c] = bf16(W_down[c] . h[t]); a wave may take
// several rows, each summed exactly as alone.  Out-of-range reads of the raw
// buffer loads return zero.
#pragma once

#include "row_dot.h"

namespace moe {
namespace {

constexpr int kSeTokens = 4;   // tokens whose operand chunks are in flight together

template <int NC>
__device__ __forceinline__ float se_dot(const u32x4 (&w)[NC], const u32x4 (&v)[NC]) {
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[c].x), as_bf16x2(v[c].x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[c].y), as_bf16x2(v[c].y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[c].z), as_bf16x2(v[c].z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[c].w), as_bf16x2(v[c].w), acc, false);
  }
  return acc;
}

// The sum of group_sum(v, 64) (lane pairs at distances 32, 16, 8, 4, 2, 1
// added in that order) without LDS-crossbar shuffles: v_permlane32_swap and
// v_permlane16_swap pair each lane with lane ^ 32 and lane ^ 16, then DPP row
// rotations by 8 and 4 and quad permutations [2,3,0,1] and [1,0,3,2].  After
// the steps at distances 32 .. d every lane of a class l mod d holds the same
// value, so a rotation by d/2 inside a 16-lane row adds the same two values
// as lane ^ (d/2); every addition has the same two operands as in group_sum
// (floating-point addition is commutative), so the result is bit for bit the
// same, in every lane.
__device__ __forceinline__ float wave_sum_xor(float v) {
  auto bits = [](float f) { return __builtin_bit_cast(uint32_t, f); };
  auto flt = [](uint32_t u) { return __builtin_bit_cast(float, u); };
  const auto p32 = __builtin_amdgcn_permlane32_swap(bits(v), bits(v), false, false);
  v = flt(p32[0]) + flt(p32[1]);
  const auto p16 = __builtin_amdgcn_permlane16_swap(bits(v), bits(v), false, false);
  v = flt(p16[0]) + flt(p16[1]);
  v = v + flt((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits(v), 0x128, 0xF, 0xF, false));   // row_ror:8
  v = v + flt((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits(v), 0x124, 0xF, 0xF, false));   // row_ror:4
  v = v + flt((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits(v), 0x4E, 0xF, 0xF, false));    // quad [2,3,0,1]
  v = v + flt((uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits(v), 0xB1, 0xF, 0xF, false));    // quad [1,0,3,2]
  return v;
}

template <int NC, int AUX>
__device__ __forceinline__ void se_load_row(__amdgpu_buffer_rsrc_t r, uint32_t row_byte, int lane, u32x4 (&dst)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
    dst[c] = __builtin_amdgcn_raw_buffer_load_b128(r, row_byte + (uint32_t)(lane + 64 * c) * 16u, 0, AUX);
}

// gate/up row r of the shared expert (r < Is), all T tokens; NC = H / 512.
// TOK tokens' activation chunks are in flight together (fewer registers for
// a smaller TOK); the sums do not depend on it.
template <int NC, int TOK = kSeTokens>
__device__ __forceinline__ void se_gate_up_row(const SharedRows& s, int r, int lane) {
  const uint32_t row_bytes = (uint32_t)s.H * 2u;
  const auto rg = make_rsrc(s.wg, (uint32_t)s.Is * row_bytes);
  const auto ru = make_rsrc(s.wu, (uint32_t)s.Is * row_bytes);
  const auto rx = make_rsrc(s.x, (uint32_t)s.T * row_bytes);
  u32x4 g[NC], u[NC];
  se_load_row<NC, kStreamAux>(rg, (uint32_t)r * row_bytes, lane, g);
  se_load_row<NC, kStreamAux>(ru, (uint32_t)r * row_bytes, lane, u);
  for (int t0 = 0; t0 < s.T; t0 += TOK) {
    u32x4 xv[TOK][NC];
#pragma unroll
    for (int j = 0; j < TOK; ++j) se_load_row<NC, 0>(rx, (uint32_t)(t0 + j) * row_bytes, lane, xv[j]);
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
      const float gs = wave_sum_xor(se_dot<NC>(g, xv[j]));
      const float us = wave_sum_xor(se_dot<NC>(u, xv[j]));
      if (lane == 0 && t0 + j < s.T) s.h[(size_t)(t0 + j) * s.Is + r] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
    }
  }
}

// down rows c0 .. c0 + RPW - 1 of the shared expert (those below H), all T
// tokens; NC = Is / 512
template <int NC, int RPW>
__device__ __forceinline__ void se_down_rows(const SharedRows& s, int c0, int lane) {
  const uint32_t row_bytes = (uint32_t)s.Is * 2u;
  const auto rd = make_rsrc(s.wd, (uint32_t)s.H * row_bytes);
  const auto rh = make_rsrc(s.h, (uint32_t)s.T * row_bytes);
  u32x4 w[RPW][NC];
#pragma unroll
  for (int q = 0; q < RPW; ++q) se_load_row<NC, kStreamAux>(rd, (uint32_t)(c0 + q) * row_bytes, lane, w[q]);
  for (int t0 = 0; t0 < s.T; t0 += kSeTokens) {
    u32x4 hv[kSeTokens][NC];
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) se_load_row<NC, 0>(rh, (uint32_t)(t0 + j) * row_bytes, lane, hv[j]);
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int j = 0; j < kSeTokens; ++j) {
        const float ys = wave_sum_xor(se_dot<NC>(w[q], hv[j]));
        if (lane == 0 && t0 + j < s.T && c0 + q < s.H)
          s.y[(size_t)(t0 + j) * s.H + c0 + q] = (uint16_t)f32_to_bf16_rne(ys);
      }
  }
}

// Rows riding along in another kernel: wave number v (counted over the
// extra workgroups) takes gate/up row v, or down rows kSeSideDownRows * v ..
constexpr int kSeSideDownRows = 4;

// workgroups of `waves` waves that the down rows take (0 when they do not ride along)
__host__ __device__ inline int se_down_side_blocks(const SharedRows& s, int waves) {
  return s.dn_nc > 0 ? ((s.H + kSeSideDownRows - 1) / kSeSideDownRows + waves - 1) / waves : 0;
}

__device__ __forceinline__ void se_gate_up_side(const SharedRows& s, int v, int lane) {
  if (v >= s.Is) return;
  switch (s.gu_nc) {
    case 1: se_gate_up_row<1>(s, v, lane); break;
    case 2: se_gate_up_row<2>(s, v, lane); break;
    case 4: se_gate_up_row<4>(s, v, lane); break;
    default: break;
  }
}

// Gate/up row v riding along in the small step's selection launch (H = 2048:
// four chunks per lane), one token at a time so that the launch keeps the
// registers of its gate/up tiles.
__device__ __forceinline__ void se_gate_up_side_small(const SharedRows& s, int v, int lane) {
  if (v < s.Is && s.gu_nc == 4) se_gate_up_row<4, 1>(s, v, lane);
}

__device__ __forceinline__ void se_down_side(const SharedRows& s, int v, int lane) {
  const int c0 = v * kSeSideDownRows;
  if (c0 >= s.H) return;
  switch (s.dn_nc) {
    case 1: se_down_rows<1, kSeSideDownRows>(s, c0, lane); break;
    case 2: se_down_rows<2, kSeSideDownRows>(s, c0, lane); break;
    default: break;
  }
}

}  // namespace
}  // namespace moe
