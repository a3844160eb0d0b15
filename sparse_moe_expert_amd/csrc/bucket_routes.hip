// moe_bucket_routes: group the R = T*k routes by expert, stable in flat route id.
//
// The counts, scan, expert ids and scatter that follow top-k in the fused
// routing kernel (page "How I forked vLLM and made Qwen3.8-Flash-Next decode
// 1.6x faster on one GPU", section "5. Hand-written kernels", paragraph
// "Fused MoE routing"), exported as the compact expert-presence list plus
// original route positions of the SM70 design note (page "Persistent
// execution for Flash-Next GGUF on SM70", section "First implementation
// boundary", step 1).  No token features are moved: only route ids.
//
// One 1024-thread workgroup (16 wavefronts):
//   1. LDS histogram of expert ids (integer atomics: the counts do not depend
//      on their order);
//   2. block-wide exclusive scans of the counts (offsets) and of the
//      "count > 0" flags (positions in the active list);
//   3. stable scatter in chunks of 1024 routes: inside a wavefront, lanes with
//      the same expert are found with one ballot per expert-id bit; the rank
//      among them plus the counts of earlier wavefronts in the chunk plus the
//      running base of the expert gives the position.  Positions never depend
//      on timing, so the result is exact and reproducible.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

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

// Exclusive scan of one value per thread across the workgroup; returns the
// exclusive prefix and writes the total to *total (all threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kWaves ? s_wave[lane] : 0;
    const int winc = wave_inclusive_scan(w);
    if (lane < kWaves) s_wave[lane] = winc - w;         // exclusive wave bases
    if (lane == kWaves - 1) s_wave[kWaves] = winc;      // total
  }
  __syncthreads();
  const int res = s_wave[wave] + inc - v;
  *total = s_wave[kWaves];
  __syncthreads();                                      // s_wave reusable
  return res;
}

__global__ __launch_bounds__(kThreads) void bucket_routes_kernel(
    const int32_t* __restrict__ topk_idx, int R, int E, int id_bits,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  __shared__ int s_base[1024];               // counts, then running bases
  __shared__ uint8_t s_wcnt[kWaves][1024];   // per-wavefront counts inside a chunk
  __shared__ int s_wave[kWaves + 1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

  for (int e = tid; e < 1024; e += kThreads) s_base[e] = 0;
  for (int i = tid; i < kWaves * 1024; i += kThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  // ids outside [0, E) violate the precondition; clamping keeps every access
  // in bounds
  for (int r = tid; r < R; r += kThreads) atomicAdd(&s_base[min(max(topk_idx[r], 0), E - 1)], 1);
  __syncthreads();

  // scans (E <= 1024: one expert per thread)
  const int c = tid < E ? s_base[tid] : 0;
  int total_routes, total_active;
  const int off = block_exclusive_scan(c, s_wave, &total_routes);
  const int apos = block_exclusive_scan(c > 0 ? 1 : 0, s_wave, &total_active);
  if (tid < E) {
    expert_count[tid] = c;
    expert_offset[tid] = off;
    if (c > 0) active_experts[apos] = tid;
    if (tid >= total_active) active_experts[tid] = -1;
    s_base[tid] = off;
  }
  if (tid == 0) {
    expert_offset[E] = total_routes;
    *n_active = total_active;
  }
  __syncthreads();

  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < R; c0 += kThreads) {
    const int r = c0 + tid;
    const bool valid = r < R;
    const int e = valid ? min(max(topk_idx[r], 0), E - 1) : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & below);
    const int wcount = __popcll(same);
    if (valid && rank == 0) s_wcnt[wave][e] = (uint8_t)wcount;
    __syncthreads();
    if (valid) {
      int pos = s_base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
      route_src[pos] = r;
      route_pos[r] = pos;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_base[e], wcount);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_bucket_routes(const int32_t* topk_idx, int T, int E, int k,
                                        int32_t* expert_count, int32_t* expert_offset,
                                        int32_t* active_experts, int32_t* n_active,
                                        int32_t* route_src, int32_t* route_pos, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_SHAPE;
  const long long R = (long long)T * k;
  if (E > 1024 || R > (1ll << 24)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !expert_count || !expert_offset || !active_experts || !n_active || !route_src ||
      !route_pos)
    return MOE_ERR_NULL_POINTER;
  if (!aligned16(topk_idx) || !aligned16(expert_count) || !aligned16(expert_offset) ||
      !aligned16(active_experts) || !aligned16(n_active) || !aligned16(route_src) ||
      !aligned16(route_pos))
    return MOE_ERR_MISALIGNED;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  bucket_routes_kernel<<<1, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      topk_idx, (int)R, E, id_bits, expert_count, expert_offset, active_experts, n_active, route_src,
      route_pos);
  return launch_status();
}
