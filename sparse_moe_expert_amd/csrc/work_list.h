// Work lists of the expert kernels, built by one workgroup of 1024 threads
// from per-expert route counts and first bucket positions: by plan_kernel
// (expert_ffn.hip) from the bucket arrays, or at the end of the one-workgroup
// bucketing kernels (routing.hip), which hold the counts already.
//
// MFMA list: every expert that takes the MFMA kernels (at least mfma_min
// routes) contributes one item per chunk of up to kWlRoutes routes,
// {expert, first bucket position, route count, 0}; items are grouped by
// route tiles of 32, the full chunks first, so that workgroups, which start
// in list order, begin with the longest items, and an expert with several
// chunks has them side by side.  plan[0] = item count; items from plan[4].
//
// Row-dot list (rd_plan): the experts with fewer routes than mfma_min (all
// experts when no MFMA kernel runs), most routes first - a counting sort
// over kRdBins bins, counts of kRdBins - 1 and more sharing the first.
// rd_list[0] = their number, rd_list[1 + i] = expert.
//
// The order inside a group or bin is that of LDS atomics: it decides which
// workgroup computes an item, never what is computed.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kWlThreads = 1024;
// Unit counters of the streaming down kernel: 8 class counters and a
// finished count, one 128-byte line each; zeroed here, before its first launch.
constexpr int kWlQueueStride = 32;
constexpr int kWlQueueInts = 9 * kWlQueueStride;
constexpr int kWlRoutes = 128;     // routes per MFMA item (the MFMA kernels' route chunk)
constexpr int kRdBins = 64;

struct WorkListShared {
  int cnt[4], base[4];
  int rh[kRdBins];
};

// Called by all kWlThreads threads of the workgroup, in uniform control flow;
// thread t brings expert e (or -1) with cnt routes from bucket position off.
__device__ __forceinline__ void build_work_lists(const WorkLists& wl, WorkListShared& sh, int e, int cnt, int off) {
  const int tid = threadIdx.x;
  if (tid < 4) sh.cnt[tid] = 0;
  if (wl.queues && tid < kWlQueueInts / kWlQueueStride) wl.queues[tid * kWlQueueStride] = 0;
  if (tid < kRdBins) sh.rh[tid] = 0;
  __syncthreads();
  int mcnt = 0, rcnt = 0;
  if (e >= 0 && cnt > 0) {
    if (wl.mfma_min > 0 && cnt >= wl.mfma_min) mcnt = cnt;
    else rcnt = cnt;
  }
  const int full = mcnt / kWlRoutes, rest = mcnt - full * kWlRoutes;
  const int rest_cls = rest > 0 ? 4 - ((rest + 31) >> 5) : -1;   // 0: four route tiles .. 3: one
  if (full > 0) atomicAdd(&sh.cnt[0], full);
  if (rest_cls >= 0) atomicAdd(&sh.cnt[rest_cls], 1);
  const int rbin = kRdBins - 1 - min(rcnt, kRdBins - 1);          // 0: most routes
  if (wl.rd_plan && rcnt > 0) atomicAdd(&sh.rh[rbin], 1);
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int c = 0; c < 4; ++c) {
      sh.base[c] = t;
      t += sh.cnt[c];
    }
    wl.plan[0] = min(t, wl.plan_max);
  }
  if (wl.rd_plan && tid < kWave) {
    // exclusive scan of the bins, one per lane
    const int v = sh.rh[tid];
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int u = __shfl_up(incl, d, kWave);
      if (tid >= d) incl += u;
    }
    sh.rh[tid] = incl - v;
    if (tid == kWave - 1) wl.rd_list[0] = incl;
  }
  __syncthreads();
  if (wl.rd_plan && rcnt > 0) wl.rd_list[1 + atomicAdd(&sh.rh[rbin], 1)] = e;
  int4* items = reinterpret_cast<int4*>(wl.plan + 4);
  if (full > 0) {
    const int b = atomicAdd(&sh.base[0], full);
    for (int c = 0; c < full; ++c)
      if (b + c < wl.plan_max) items[b + c] = make_int4(e, off + c * kWlRoutes, kWlRoutes, 0);
  }
  if (rest_cls >= 0) {
    const int b = atomicAdd(&sh.base[rest_cls], 1);
    if (b < wl.plan_max) items[b] = make_int4(e, off + full * kWlRoutes, rest, 0);
  }
}

}  // namespace moe
