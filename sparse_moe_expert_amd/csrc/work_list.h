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
// When chunks of half that size (64 routes) still make at most
// wl.split_items items, the gate/up list's chunks are halved: a batch that
// fills the device's workgroup slots once (256 Zipf-routed tokens) then has
// no item of three or four route tiles, whose step time set the span of the
// whole launch.  The down kernels' list (plan_down, same layout) keeps
// chunks of up to kWlRoutes routes: their row tiles outnumber the slots
// already, and halved items would add a partial round.
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
  int cnt_d[4], base_d[4];          // the down list's classes
  int rh[kRdBins];
  int n_half;                       // items with chunks of kWlRoutes / 2 routes
};

// Items of one expert's mcnt routes in chunks of cs: `full` whole chunks and
// a rest; their classes (0: four route tiles .. 3: one) and list slots.
__device__ __forceinline__ void wl_chunks(int mcnt, int cs, int& full, int& rest, int& full_cls, int& rest_cls) {
  full = mcnt / cs;
  rest = mcnt - full * cs;
  full_cls = 4 - cs / 32;
  rest_cls = rest > 0 ? 4 - ((rest + 31) >> 5) : -1;
}

__device__ __forceinline__ void wl_write(int4* items, int plan_max, int b_full, int b_rest, int e, int off, int cs,
                                         int full, int rest, int rest_cls) {
  for (int c = 0; c < full; ++c)
    if (b_full + c < plan_max) items[b_full + c] = make_int4(e, off + c * cs, cs, 0);
  if (rest_cls >= 0 && b_rest < plan_max) items[b_rest] = make_int4(e, off + full * cs, rest, 0);
}

// Called by all kWlThreads threads of the workgroup, in uniform control flow;
// thread t brings expert e (or -1) with cnt routes from bucket position off.
__device__ __forceinline__ void build_work_lists(const WorkLists& wl, WorkListShared& sh, int e, int cnt, int off) {
  const int tid = threadIdx.x;
  if (tid < 4) {
    sh.cnt[tid] = 0;
    sh.cnt_d[tid] = 0;
  }
  if (tid == 0) sh.n_half = 0;
  if (wl.queues && tid < kWlQueueInts / kWlQueueStride) wl.queues[tid * kWlQueueStride] = 0;
  if (tid < kRdBins) sh.rh[tid] = 0;
  __syncthreads();
  int mcnt = 0, rcnt = 0;
  if (e >= 0 && cnt > 0) {
    if (wl.mfma_min > 0 && cnt >= wl.mfma_min) mcnt = cnt;
    else rcnt = cnt;
  }
  constexpr int kHalf = kWlRoutes / 2;
  if (wl.split_items > 0 && mcnt > 0) atomicAdd(&sh.n_half, (mcnt + kHalf - 1) / kHalf);
  __syncthreads();
  const int cs = (wl.split_items > 0 && sh.n_half <= wl.split_items) ? kHalf : kWlRoutes;   // uniform
  int full, rest, full_cls, rest_cls;
  wl_chunks(mcnt, cs, full, rest, full_cls, rest_cls);
  if (full > 0) atomicAdd(&sh.cnt[full_cls], full);
  if (rest_cls >= 0) atomicAdd(&sh.cnt[rest_cls], 1);
  int full_d, rest_d, full_cls_d, rest_cls_d;
  wl_chunks(mcnt, kWlRoutes, full_d, rest_d, full_cls_d, rest_cls_d);
  if (wl.plan_down) {
    if (full_d > 0) atomicAdd(&sh.cnt_d[full_cls_d], full_d);
    if (rest_cls_d >= 0) atomicAdd(&sh.cnt_d[rest_cls_d], 1);
  }
  const int rbin = kRdBins - 1 - min(rcnt, kRdBins - 1);          // 0: most routes
  if (wl.rd_plan && rcnt > 0) atomicAdd(&sh.rh[rbin], 1);
  __syncthreads();
  if (tid == 0) {
    int t = 0, td = 0;
    for (int c = 0; c < 4; ++c) {
      sh.base[c] = t;
      t += sh.cnt[c];
      sh.base_d[c] = td;
      td += sh.cnt_d[c];
    }
    wl.plan[0] = min(t, wl.plan_max);
    if (wl.plan_down) wl.plan_down[0] = min(td, wl.plan_max);
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
  if (full > 0 || rest_cls >= 0) {
    const int bf = full > 0 ? atomicAdd(&sh.base[full_cls], full) : 0;
    const int br = rest_cls >= 0 ? atomicAdd(&sh.base[rest_cls], 1) : 0;
    wl_write(reinterpret_cast<int4*>(wl.plan + 4), wl.plan_max, bf, br, e, off, cs, full, rest, rest_cls);
  }
  if (wl.plan_down && (full_d > 0 || rest_cls_d >= 0)) {
    const int bf = full_d > 0 ? atomicAdd(&sh.base_d[full_cls_d], full_d) : 0;
    const int br = rest_cls_d >= 0 ? atomicAdd(&sh.base_d[rest_cls_d], 1) : 0;
    wl_write(reinterpret_cast<int4*>(wl.plan_down + 4), wl.plan_max, bf, br, e, off, kWlRoutes, full_d, rest_d,
             rest_cls_d);
  }
}

}  // namespace moe
