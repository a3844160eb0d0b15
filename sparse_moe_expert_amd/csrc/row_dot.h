// Device building blocks of the NVFP4 row-dot kernels (gfx950).
//
// A wavefront reads whole weight rows: Lr lanes share a row and each lane
// reads one 16-byte chunk of e2m1 codes (32 values) plus the chunk's two e4m3
// scales.  Byte pairs become bf16 with v_cvt_scalef32_pk_bf16_fp4 (exact at
// scale 1), v_dot2 multiplies them with the operand (activations or the
// intermediate) in bf16 pairs with fp32 accumulation, one scale multiplies
// each 16-value block, and a row's partial sums are added across its lanes
// with DPP row operations and v_permlane{16,32}_swap in a fixed order.
#pragma once

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
// Cache policy of the row-dot weight streams: non-temporal.  Each of these
// loads consumes whole cache lines and every weight and scale byte of a step
// is read once, so they are marked as streaming and do not displace the small
// reused data (routing metadata, activations, h) from the caches; measured on
// gfx950 this shortens the decode step by ~10%.
constexpr int kStreamAux = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

// Buffer resource over [base, base + bytes): loads outside it return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

// 1.0f in a scalar register whose value the optimiser cannot see (no
// instruction).  Per-route loops pass it as the scale operand of the weight
// conversions, so those are not hoisted out of the loop (which would keep
// every converted value live at once), while the weight registers
// themselves stay untouched: an asm that rewrote them would make the
// register allocator copy them, and each copy waits for its load.
__device__ __forceinline__ float opaque_one() {
  float v = 1.0f;
  asm volatile("" : "+s"(v));
  return v;
}

// One 16-byte chunk (32 NVFP4 values, two scale blocks) dotted with an
// operand chunk xr (operand elements 2i, 2i+1 as bf16x2 in xr[i]); adds
// sum_block(scale * sum(code * operand)) to acc.  `one` is 1.0f (see
// opaque_one).
__device__ __forceinline__ float dot_chunk(const uint4 codes, uint32_t s2, const uint32_t (&xr)[16], float acc,
                                           float one) {
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 1);
  const uint32_t c[4] = {codes.x, codes.y, codes.z, codes.w};
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    p0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(c[q], one), as_bf16x2(xr[4 * q + 0]), p0, false);
    p0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(c[q], one), as_bf16x2(xr[4 * q + 1]), p0, false);
    p0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(c[q], one), as_bf16x2(xr[4 * q + 2]), p0, false);
    p0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(c[q], one), as_bf16x2(xr[4 * q + 3]), p0, false);
  }
#pragma unroll
  for (int q = 2; q < 4; ++q) {
    p1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(c[q], one), as_bf16x2(xr[4 * q + 0]), p1, false);
    p1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(c[q], one), as_bf16x2(xr[4 * q + 1]), p1, false);
    p1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(c[q], one), as_bf16x2(xr[4 * q + 2]), p1, false);
    p1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(c[q], one), as_bf16x2(xr[4 * q + 3]), p1, false);
  }
  acc = fmaf(p0, s0, acc);
  return fmaf(p1, s1, acc);
}

// Load the 64-byte operand chunk `chunk` of a bf16 row into 16 dwords.
__device__ __forceinline__ void load_operand_chunk(const uint16_t* row, int chunk, uint32_t (&dst)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(row + (size_t)chunk * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    dst[4 * q + 0] = v.x; dst[4 * q + 1] = v.y; dst[4 * q + 2] = v.z; dst[4 * q + 3] = v.w;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane row (fixed order); every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x124>(v);   // row_ror:4
  v = dpp_add<0x128>(v);   // row_ror:8
  return v;
}

__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }

// a0..a3 hold row sums (uniform within each 16-lane row).  Returns a value
// whose row r holds a_r summed over all four rows (v_permlane32_swap swaps the
// upper rows of its first operand with the lower rows of its second;
// v_permlane16_swap swaps odd rows of the first with even rows of the second).
__device__ __forceinline__ float rows_scatter4(float a0, float a1, float a2, float a3) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(fbits(a0), fbits(a2), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(fbits(a1), fbits(a3), false, false);
  const float b02 = bitsf(s02[0]) + bitsf(s02[1]);
  const float b13 = bitsf(s13[0]) + bitsf(s13[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(fbits(b02), fbits(b13), false, false);
  return bitsf(t[0]) + bitsf(t[1]);
}

// Lane geometry of one projection.  LR: lanes per row known at compile time
// (64 for rows of 2048 values, 16 for rows of 512), or 0 for a runtime value.
template <int LR, int UNITS>
struct Geo {
  int lr, rpw, sub, sl, rpt, tiles, wave;
  __device__ Geo(int lr_rt, int rows_total) {
    const int lane = threadIdx.x & (kWave - 1);
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lr = LR ? LR : lr_rt;
    rpw = kWave / lr;
    sub = lane / lr;
    sl = lane & (lr - 1);
    rpt = kWavesPerBlock * rpw * UNITS;
    tiles = (rows_total + rpt - 1) / rpt;
  }
  // first row of unit u for this wave (wave-uniform); the lane's row adds sub
  __device__ int row0(int tile, int u) const { return tile * rpt + (u * kWavesPerBlock + wave) * rpw; }
};

}  // namespace
}  // namespace moe
