// Dense BF16 shared expert: y_t = W_down (SiLU(W_gate x_t) * (W_up x_t)) for
// every token (page "How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x
// faster on one GPU", section "2. FP8 for the dense layers": shared experts
// stay BF16; page "Persistent execution for Flash-Next GGUF on SM70", section
// "Opportunity sized from the actual routes": their work runs beside the
// routed experts').  Decode-sized batches make both projections matrix-vector
// products, bound by the weight bytes (3 * H * Is * 2).
//
// Two kernels, one wavefront per weight row.  Gate/up: wave r holds rows r of
// W_gate and W_up in registers (64 lanes x H/64 values, 16-byte loads), takes
// the tokens four at a time (their x chunks issued together), multiplies
// bf16 pairs with v_dot2_f32_bf16 into fp32, sums the 64 lanes in a fixed
// butterfly order and writes h[t, r] = bf16(SiLU(g) * u) to the workspace.
// Down: wave c holds row c of W_down and writes y[t, c] = bf16(W_down[c] . h[t])
// the same way.  Every load is a raw buffer load over the tensor it reads
// (out-of-range reads return zero), every sum has a fixed order: results are
// bitwise reproducible.
#include "row_dot.h"

namespace moe {
namespace {

constexpr int kSeThreads = 256;       // four waves, one weight row each
constexpr int kSeWaves = kSeThreads / kWave;
constexpr int kSeTokens = 4;          // tokens whose operand chunks are in flight together

// dot of NC 16-byte chunks (8 bf16 each) of a weight row with the same
// chunks of an operand row, fp32
template <int NC>
__device__ __forceinline__ float dot_chunks(const u32x4 (&w)[NC], const u32x4 (&v)[NC]) {
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

// Lane l's chunk c of a row of K values covers values 8*(l + 64c) .. +8:
// a wave reads 1 KB contiguous per chunk.
template <int NC, int AUX>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t r, uint32_t row_byte, int lane, u32x4 (&dst)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
    dst[c] = __builtin_amdgcn_raw_buffer_load_b128(r, row_byte + (uint32_t)(lane + 64 * c) * 16u, 0, AUX);
}

template <int NC>
__global__ __launch_bounds__(kSeThreads) void shared_gate_up_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wg,
                                                                    const uint16_t* __restrict__ wu, int T, int H,
                                                                    int Is, uint16_t* __restrict__ h) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * kSeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= Is) return;
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const auto rg = make_rsrc(wg, (uint32_t)Is * row_bytes);
  const auto ru = make_rsrc(wu, (uint32_t)Is * row_bytes);
  const auto rx = make_rsrc(x, (uint32_t)T * row_bytes);
  u32x4 g[NC], u[NC];
  load_row<NC, kStreamAux>(rg, (uint32_t)r * row_bytes, lane, g);
  load_row<NC, kStreamAux>(ru, (uint32_t)r * row_bytes, lane, u);
  for (int t0 = 0; t0 < T; t0 += kSeTokens) {
    u32x4 xv[kSeTokens][NC];
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) load_row<NC, 0>(rx, (uint32_t)(t0 + j) * row_bytes, lane, xv[j]);
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) {
      const float gs = group_sum(dot_chunks<NC>(g, xv[j]), kWave);
      const float us = group_sum(dot_chunks<NC>(u, xv[j]), kWave);
      if (lane == 0 && t0 + j < T) h[(size_t)(t0 + j) * Is + r] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
    }
  }
}

template <int NC>
__global__ __launch_bounds__(kSeThreads) void shared_down_kernel(const uint16_t* __restrict__ h,
                                                                 const uint16_t* __restrict__ wd, int T, int H,
                                                                 int Is, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = blockIdx.x * kSeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (c >= H) return;
  const uint32_t row_bytes = (uint32_t)Is * 2u;
  const auto rd = make_rsrc(wd, (uint32_t)H * row_bytes);
  const auto rh = make_rsrc(h, (uint32_t)T * row_bytes);
  u32x4 w[NC];
  load_row<NC, kStreamAux>(rd, (uint32_t)c * row_bytes, lane, w);
  for (int t0 = 0; t0 < T; t0 += kSeTokens) {
    u32x4 hv[kSeTokens][NC];
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) load_row<NC, 0>(rh, (uint32_t)(t0 + j) * row_bytes, lane, hv[j]);
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) {
      const float ys = group_sum(dot_chunks<NC>(w, hv[j]), kWave);
      if (lane == 0 && t0 + j < T) y[(size_t)(t0 + j) * H + c] = (uint16_t)f32_to_bf16_rne(ys);
    }
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace
}  // namespace moe

extern "C" size_t moe_shared_expert_workspace_size(int T, int H, int Is) {
  (void)H;
  if (T <= 0 || Is <= 0) return 0;
  return moe::align256((size_t)T * (size_t)Is * 2);
}

extern "C" moe_status moe_shared_expert(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                                        const uint16_t* w_down, int T, int H, int Is, void* workspace,
                                        size_t workspace_bytes, uint16_t* y, void* stream) {
  using namespace moe;
  if (T < 0 || H < 32 || Is < 32 || H % 32 != 0 || Is % 32 != 0) return MOE_ERR_INVALID_SHAPE;
  // one to eight 16-byte chunks per lane: rows of 512 .. 4096 values in steps of 512
  if (H % 512 != 0 || Is % 512 != 0 || H > 4096 || Is > 4096 || T > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, w_up, w_down, workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  if (workspace_bytes < moe_shared_expert_workspace_size(T, H, Is)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  // one buffer resource per tensor: byte counts must fit 31 bits
  if ((size_t)T * H * 2 >= 0x80000000ull || (size_t)Is * H * 2 >= 0x80000000ull) return MOE_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = static_cast<uint16_t*>(workspace);
  const unsigned g1 = (unsigned)((Is + kSeWaves - 1) / kSeWaves), g2 = (unsigned)((H + kSeWaves - 1) / kSeWaves);
  switch (H / 512) {
    case 1: shared_gate_up_kernel<1><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 2: shared_gate_up_kernel<2><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 3: shared_gate_up_kernel<3><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 4: shared_gate_up_kernel<4><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 5: shared_gate_up_kernel<5><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 6: shared_gate_up_kernel<6><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    case 7: shared_gate_up_kernel<7><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
    default: shared_gate_up_kernel<8><<<g1, kSeThreads, 0, s>>>(x, w_gate, w_up, T, H, Is, h); break;
  }
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  switch (Is / 512) {
    case 1: shared_down_kernel<1><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 2: shared_down_kernel<2><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 3: shared_down_kernel<3><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 4: shared_down_kernel<4><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 5: shared_down_kernel<5><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 6: shared_down_kernel<6><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    case 7: shared_down_kernel<7><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
    default: shared_down_kernel<8><<<g2, kSeThreads, 0, s>>>(h, w_down, T, H, Is, y); break;
  }
  return launch_status();
}
