// One-workgroup bucketing (1024 threads) of R routes by expert: per-expert
// counts, exclusive offsets, the ascending active list and the stable
// scatter (route order within each expert).  Shared by the routing kernels
// and by the small-batch down/unroute launch that buckets the routes its
// gate/up launch selected.
#pragma once

#include "select.h"
#include "work_list.h"

namespace moe {
namespace {

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / kWave;

// Exclusive scan of one value per thread across the workgroup; returns the
// exclusive prefix and writes the total to *total (all threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kBucketWaves ? s_wave[lane] : 0;
    const int winc = wave_inclusive_scan(w);
    if (lane < kBucketWaves) s_wave[lane] = winc - w;         // exclusive wave bases
    if (lane == kBucketWaves - 1) s_wave[kBucketWaves] = winc;      // total
  }
  __syncthreads();
  const int res = s_wave[wave] + inc - v;
  *total = s_wave[kBucketWaves];
  __syncthreads();                                      // s_wave reusable
  return res;
}

struct BucketShared {
  int base[1024];                    // counts, then running bases
  uint8_t wcnt[kBucketWaves][1024];  // per-wavefront counts inside a chunk
  int wave_tot[kBucketWaves + 1];
  WorkListShared wl;
};
static_assert(kBucketThreads == kWlThreads, "the bucketing workgroup builds the work lists");

// Bucket R routes whose expert ids are ids[0..R) (global or LDS).
// With wl.plan set it also builds the expert kernels' work lists.
__device__ __forceinline__ void bucket_block(const int32_t* ids, int R, int E, BucketShared& sh,
                                             int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
                                             int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
                                             int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos,
                                             const WorkLists& wl) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < 1024; e += kBucketThreads) sh.base[e] = 0;
  for (int i = tid; i < kBucketWaves * 1024 / 4; i += kBucketThreads) reinterpret_cast<int*>(&sh.wcnt[0][0])[i] = 0;
  __syncthreads();
  // ids outside [0, E) violate the precondition; clamping keeps every access
  // in bounds
  for (int r = tid; r < R; r += kBucketThreads) atomicAdd(&sh.base[min(max(ids[r], 0), E - 1)], 1);
  __syncthreads();

  // scans (E <= 1024: one expert per thread) of the counts and of the
  // count > 0 flags - one scan of both packed in one int while R < 2^16
  const int c = tid < E ? sh.base[tid] : 0;
  int off, apos, total_routes, total_active;
  if (R < (1 << 16)) {
    int total;
    const int scan = block_exclusive_scan(c + ((c > 0) << 16), sh.wave_tot, &total);
    off = scan & 0xFFFF;
    apos = scan >> 16;
    total_routes = total & 0xFFFF;
    total_active = total >> 16;
  } else {
    off = block_exclusive_scan(c, sh.wave_tot, &total_routes);
    apos = block_exclusive_scan(c > 0 ? 1 : 0, sh.wave_tot, &total_active);
  }
  if (tid < E) {
    expert_count[tid] = c;
    expert_offset[tid] = off;
    if (c > 0) active_experts[apos] = tid;
    if (tid >= total_active) active_experts[tid] = -1;
    sh.base[tid] = off;
  }
  if (tid == 0) {
    expert_offset[E] = total_routes;
    *n_active = total_active;
  }
  if (wl.plan) build_work_lists(wl, sh.wl, tid < E ? tid : -1, c, off);   // uniform: a kernel argument
  __syncthreads();

  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < R; c0 += kBucketThreads) {
    const int r = c0 + tid;
    const bool valid = r < R;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {                // ids are below 1024
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & below);
    const int wcount = __popcll(same);
    if (valid && rank == 0) sh.wcnt[wave][e] = (uint8_t)wcount;
    __syncthreads();
    if (valid) {
      int pos = sh.base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += sh.wcnt[w][e];
      route_src[pos] = r;
      route_pos[r] = pos;
    }
    if (c0 + kBucketThreads >= R) break;          // last chunk: no bases to carry
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&sh.base[e], wcount);
      sh.wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe
