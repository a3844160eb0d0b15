// Routing: moe_route_topk, moe_bucket_routes and their fused form
// moe_route_bucket.
//
// Selection follows the fused MoE routing kernel's rule (page "How I forked
// vLLM and made Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section
// "5. Hand-written kernels", paragraph "Fused MoE routing"): repeated arg-max
// over the scores with the lowest expert id winning ties, lanes holding
// contiguous experts read with vector loads.  The SM70 note's router section
// states the same tie rule for its repeated-maxima selection (page
// "Persistent execution for Flash-Next GGUF on SM70", section "Router:
// selection and expert-task production").  Bucketing is the counts, scan,
// expert ids and scatter that follow top-k in the fused routing kernel,
// exported as the compact expert-presence list plus original route positions
// of the SM70 note (section "First implementation boundary", step 1).  The
// same page paragraph describes one workgroup doing all of it for small
// batches; moe_route_bucket does that here up to 16 tokens.
//
// Selection (gfx950, select.h): one 64-lane wavefront per token, k rounds of
// a wave-wide arg-max over order-preserving integer keys.  A selection is a
// chain of dependent wave operations, so it runs at full speed only with
// few waves per SIMD; batches of more than 16 tokens therefore select in a
// kernel of four tokens per workgroup spread over the chip, and bucket in a
// second one-workgroup kernel.
//
// Bucketing (one 1024-thread workgroup): LDS histogram of expert ids
// (integer atomics: counts do not depend on their order), block-wide
// exclusive scans of the counts and of the "count > 0" flags, then a stable
// scatter in chunks of 1024 routes: lanes of a wavefront with the same expert
// are found with one ballot per id bit; rank among them + counts of earlier
// wavefronts in the chunk + the expert's running base gives the position.
// Positions never depend on timing, so the result is exact and reproducible.
// Batches of 1025 to 65536 routes bucket in one launch of one such
// workgroup per 1024-route chunk (bucket_chunked_kernel), larger ones in
// three launches over a scratch array of per-chunk counts.
#include "router_rows.h"
#include "bucket_block.h"
#include "select.h"
#include "shared_rows.h"
#include "work_list.h"

namespace moe {
namespace {

// The selecting kernels are also built with k fixed at this value (the
// configured top-10), which unrolls the selection rounds; other k use the
// loop.
constexpr int kUnrolledK = 10;

template <int V, int KC>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                           // whole wavefront leaves together
  int e;
  float w;
  select_token<V, KC>(logits + (size_t)t * E, bias, E, k, lane, e, w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = e;
    topk_w[(size_t)t * k + lane] = w;
  }
}

__global__ __launch_bounds__(kBucketThreads) void bucket_routes_kernel(
    const int32_t* __restrict__ topk_idx, int R, int E,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos, WorkLists wl) {
  __shared__ BucketShared sh;
  bucket_block(topk_idx, R, E, sh, expert_count, expert_offset, active_experts, n_active, route_src,
               route_pos, wl);
}

// Bucketing of batches beyond kChunkedMaxRoutes routes in parallel (three
// kernels over chunks of kBucketThreads routes), with a caller-provided
// scratch array counts[C][E]:
//   bucket_count_kernel    chunk c: per-expert route counts of the chunk
//   bucket_scan_kernel     one workgroup: for every expert the exclusive
//                          prefix of its counts over the chunks (in place),
//                          its total, offset and active position
//   bucket_scatter_kernel  chunk c: position = expert offset + prefix of
//                          earlier chunks + rank inside the chunk (ballots)
// The positions are the same as the one-workgroup bucketing's: a route's
// rank among the routes of its expert in route order.
constexpr int kChunkMinChunks = 8;             // batches of more chunks than this take the parallel path

__global__ __launch_bounds__(kBucketThreads) void bucket_count_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                      int32_t* __restrict__ counts) {
  __shared__ int s_cnt[1024];
  const int tid = threadIdx.x, c = blockIdx.x;
  s_cnt[tid] = 0;
  __syncthreads();
  const int r = c * kBucketThreads + tid;
  if (r < R) atomicAdd(&s_cnt[min(max(ids[r], 0), E - 1)], 1);    // integer counts: order-free
  __syncthreads();
  if (tid < E) counts[(size_t)c * E + tid] = s_cnt[tid];
}

__global__ __launch_bounds__(kBucketThreads) void bucket_scan_kernel(
    int32_t* __restrict__ counts, int C, int E, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    WorkLists wl) {
  __shared__ int s_wave[kBucketWaves + 1];
  __shared__ WorkListShared s_wl;
  const int tid = threadIdx.x;
  int run = 0;
  if (tid < E) {
    constexpr int kB = 8;                      // chunk counts fetched together
    for (int c0 = 0; c0 < C; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) v[j] = c0 + j < C ? counts[(size_t)(c0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (c0 + j < C) {
          counts[(size_t)(c0 + j) * E + tid] = run;
          run += v[j];
        }
    }
  }
  int total_routes, total_active;
  const int off = block_exclusive_scan(run, s_wave, &total_routes);
  const int apos = block_exclusive_scan(run > 0 ? 1 : 0, s_wave, &total_active);
  if (tid < E) {
    expert_count[tid] = run;
    expert_offset[tid] = off;
    if (run > 0) active_experts[apos] = tid;
    if (tid >= total_active) active_experts[tid] = -1;
  }
  if (tid == 0) {
    expert_offset[E] = total_routes;
    *n_active = total_active;
  }
  if (wl.plan) build_work_lists(wl, s_wl, tid < E ? tid : -1, run, off);   // uniform: a kernel argument
}

__global__ __launch_bounds__(kBucketThreads) void bucket_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int id_bits, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ expert_offset, int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  __shared__ int s_base[1024];
  __shared__ uint8_t s_wcnt[kBucketWaves][1024];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6, c = blockIdx.x;
  if (tid < E) s_base[tid] = expert_offset[tid] + counts[(size_t)c * E + tid];
  for (int i = tid; i < kBucketWaves * 1024 / 4; i += kBucketThreads) reinterpret_cast<int*>(&s_wcnt[0][0])[i] = 0;
  const int r = c * kBucketThreads + tid;
  const bool valid = r < R;
  const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  int rank = __popcll(same & ((1ull << lane) - 1ull));
  __syncthreads();                             // s_wcnt cleared, s_base set
  if (valid && rank == 0) s_wcnt[wave][e] = (uint8_t)__popcll(same);
  __syncthreads();
  if (valid) {
    for (int w = 0; w < wave; ++w) rank += s_wcnt[w][e];
    const int pos = s_base[e] + rank;
    route_src[pos] = r;
    route_pos[r] = pos;
  }
}

// Bucketing of batches of 1025 to kChunkedMaxRoutes routes in one launch of
// one workgroup per chunk of kBucketThreads routes, without scratch memory.
// Workgroup c counts the expert ids of the whole batch (160 KB at 40960
// routes, read from L2) into two LDS histograms - every route, and the routes
// before its chunk - so that it knows each expert's total, offset and the
// number of its routes in earlier chunks without waiting for another
// workgroup; integer atomics make both histograms independent of order.  It
// then ranks its own chunk's routes like the one-workgroup bucketing
// (ballots per id bit inside a wavefront, counts of earlier wavefronts) and
// scatters them.  Workgroup 0 also writes the per-expert arrays and the work
// lists.  The positions equal the one-workgroup bucketing's.
constexpr int kChunkedMaxRoutes = 1 << 16;
constexpr int kChunkedGroups = kChunkedMaxRoutes / 4 / kBucketThreads;   // 16-byte id groups per thread
static_assert(kChunkedGroups * 4 * kBucketThreads >= kChunkedMaxRoutes, "one load pass covers every id");

struct ChunkedShared {
  int tot[1024];
  int pre[1024];
  uint8_t wcnt[kBucketWaves][1024];
  int wave_tot[kBucketWaves + 1];
  WorkListShared wl;
};

__global__ __launch_bounds__(kBucketThreads) void bucket_chunked_kernel(
    const int32_t* __restrict__ ids, int R, int E, int id_bits, int32_t* __restrict__ expert_count,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos, WorkLists wl) {
  __shared__ ChunkedShared sh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6, c = blockIdx.x;
  sh.tot[tid] = 0;
  for (int i = tid; i < kBucketWaves * 1024 / 4; i += kBucketThreads) reinterpret_cast<int*>(&sh.wcnt[0][0])[i] = 0;
  __syncthreads();
  // ids outside [0, E) violate the precondition; clamping keeps every access
  // in bounds.  Thread t takes the whole 16-byte groups t + 1024 u, all of
  // them loaded before the first atomic (one round trip instead of one per
  // pass; the resource ends at the last whole group, past which loads read
  // zeros and are not counted), and threads 0..2 the last R % 4 routes.  The
  // routes before c * 1024 (the earlier chunks, whole groups) are counted
  // first; the histogram at that point is the prefix, copied before the rest
  // is counted.
  const int groups = R / 4;
  const auto rid = make_rsrc(ids, (uint32_t)groups * 16u);
  const int own_group = c * (kBucketThreads / 4);
  u32x4 v[kChunkedGroups];
#pragma unroll
  for (int u = 0; u < kChunkedGroups; ++u)
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rid, (uint32_t)(u * kBucketThreads + tid) * 16u, 0, 0);
  const int rt = groups * 4 + tid;
  const int e_tail = rt < R ? min(max(ids[rt], 0), E - 1) : -1;
#pragma unroll
  for (int u = 0; u < kChunkedGroups; ++u) {
    const int g = u * kBucketThreads + tid;
    if (g < min(groups, own_group)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&sh.tot[min(max((int)v[u][i], 0), E - 1)], 1);
    }
  }
  __syncthreads();
  sh.pre[tid] = sh.tot[tid];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kChunkedGroups; ++u) {
    const int g = u * kBucketThreads + tid;
    if (g >= own_group && g < groups) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&sh.tot[min(max((int)v[u][i], 0), E - 1)], 1);
    }
  }
  if (e_tail >= 0) atomicAdd(&sh.tot[e_tail], 1);   // the tail lies in the last chunk, never before c
  __syncthreads();
  const int cnt = tid < E ? sh.tot[tid] : 0;
  int off, apos, total_routes, total_active;
  if (R < (1 << 16)) {
    int total;
    const int scan = block_exclusive_scan(cnt + ((cnt > 0) << 16), sh.wave_tot, &total);
    off = scan & 0xFFFF;
    apos = scan >> 16;
    total_routes = total & 0xFFFF;
    total_active = total >> 16;
  } else {
    off = block_exclusive_scan(cnt, sh.wave_tot, &total_routes);
    apos = block_exclusive_scan(cnt > 0 ? 1 : 0, sh.wave_tot, &total_active);
  }
  if (c == 0) {                                   // uniform in the workgroup
    if (tid < E) {
      expert_count[tid] = cnt;
      expert_offset[tid] = off;
      if (cnt > 0) active_experts[apos] = tid;
      if (tid >= total_active) active_experts[tid] = -1;
    }
    if (tid == 0) {
      expert_offset[E] = total_routes;
      *n_active = total_active;
    }
    if (wl.plan) build_work_lists(wl, sh.wl, tid < E ? tid : -1, cnt, off);   // uniform: a kernel argument
  }
  if (tid < E) sh.pre[tid] += off;               // first position of the expert's routes in this chunk
  // this chunk's routes: rank = earlier routes of the same expert in the chunk
  const int r = c * kBucketThreads + tid;
  const bool valid = r < R;
  const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  int rank = __popcll(same & ((1ull << lane) - 1ull));
  __syncthreads();                                // sh.pre holds the bases
  if (valid && rank == 0) sh.wcnt[wave][e] = (uint8_t)__popcll(same);
  __syncthreads();
  if (valid) {
    for (int w = 0; w < wave; ++w) rank += sh.wcnt[w][e];
    const int pos = sh.pre[e] + rank;
    route_src[pos] = r;
    route_pos[r] = pos;
  }
}

// Route and bucket a batch of up to 16 tokens in one workgroup of NT threads
// (512 when E <= 512 and T <= 8: fewer waves to meet at each barrier, else
// 1024): wavefront w selects token w; bucketing is an LDS histogram, one packed
// scan over one expert per thread (route offsets in the low half,
// active-expert positions in the high half), and a stable scatter whose rank
// is the number of earlier routes to the same expert (ballots per id bit
// inside a 64-route group, per-expert counts of earlier groups).
constexpr int kSmallMaxTokens = 16;
constexpr int kSmallMaxRoutes = 256;
// Up to 512 experts (eight keys per lane): sorting sixteen 64-bit keys per
// lane takes ~146 registers, more than a 1024-thread workgroup may hold, so
// larger E select in route_topk_kernel (no register cap) and bucket apart.
constexpr int kSmallMaxExperts = 8 * kWave;

// shared-expert gate/up rows per extra workgroup of the small routing kernel
// (two per 512-thread workgroup, two of which fit a compute unit; four per
// 1024-thread one, one of which fits): every such workgroup resident at once
template <int NT>
constexpr int kSmallSideWaves = NT >= 1024 ? 4 : 2;

// The routing and bucketing of the whole batch by the NT threads of one
// workgroup (every thread calls it).
template <int V, int KC, int NT>
__device__ __forceinline__ void route_bucket_block(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  __shared__ int s_cnt[NT];
  __shared__ int s_ids[kSmallMaxRoutes];
  constexpr int NW = NT / kWave;
  __shared__ int s_wt[NW];
  __shared__ uint8_t s_wcnt[kSmallMaxRoutes / kWave][NT];     // routes per expert in each 64-route group
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int R = T * k;
  s_cnt[tid] = 0;
  for (int i = tid; i < kSmallMaxRoutes / kWave * NT / 4; i += NT) reinterpret_cast<int*>(&s_wcnt[0][0])[i] = 0;
  if (wave < T) {
    int e;
    float w;
    select_token<V, KC>(logits + (size_t)wave * E, bias, E, k, lane, e, w);
    if (lane < k) {
      topk_idx[(size_t)wave * k + lane] = e;
      topk_w[(size_t)wave * k + lane] = w;
      s_ids[wave * k + lane] = e;
    }
  }
  __syncthreads();
  // counts (LDS integer atomics: order-free) and, within each 64-route
  // group, the stable rank of a route among the group's routes to the same
  // expert (one ballot per id bit; ids are below 1024), both before the
  // next barrier
  const bool valid = tid < R;
  int rank = 0, e = 0;
  if (wave * kWave < R) {
    e = valid ? s_ids[tid] : 0;
    if (valid) atomicAdd(&s_cnt[e], 1);
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    rank = __popcll(same & ((1ull << lane) - 1ull));
    if (valid && rank == 0) s_wcnt[wave][e] = (uint8_t)__popcll(same);
  }
  __syncthreads();
  const int c = s_cnt[tid];                          // expert tid
  // exclusive scan over the experts of (count, count > 0) packed in one int
  const int v = c + ((c > 0) << 16);
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wt[wave] = inc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = s_wt[w];
    base += (w < wave) ? t : 0;
    total += t;
  }
  const int scan = base + inc - v;
  const int off = scan & 0xFFFF, apos = scan >> 16;
  const int total_active = total >> 16;
  if (tid < E) {
    expert_count[tid] = c;
    expert_offset[tid] = off;
    if (c > 0) active_experts[apos] = tid;
    if (tid >= total_active) active_experts[tid] = -1;
    s_cnt[tid] = off;                              // base for the scatter
  }
  if (tid == 0) {
    expert_offset[E] = total & 0xFFFF;
    *n_active = total_active;
  }
  __syncthreads();
  if (valid) {
    for (int w = 0; w < wave; ++w) rank += s_wcnt[w][e];
    const int pos = s_cnt[e] + rank;
    route_src[pos] = tid;
    route_pos[tid] = pos;
  }
}

template <int V, int KC, int NT>
__global__ __launch_bounds__(NT) void route_bucket_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos, SharedRows sr) {
  // workgroups after the first compute rows of a shared expert's gate/up
  // (moe_step_shared), one per wave, while the first one routes; only the
  // first kSmallSideWaves<NT> waves of such a workgroup take rows, which
  // spreads the weight and activation reads over more compute units
  if (blockIdx.x > 0) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < kSmallSideWaves<NT>)
      se_gate_up_side(sr, (int)(blockIdx.x - 1) * kSmallSideWaves<NT> + w, threadIdx.x & (kWave - 1));
    return;
  }
  route_bucket_block<V, KC, NT>(logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset,
                                active_experts, n_active, route_src, route_pos);
}

// The router projection, selection and bucketing of a small batch in one
// launch (page "Persistent execution for Flash-Next GGUF on SM70", section
// "Router: selection and expert-task production": the projection's results
// span many workgroups, so a fused kernel needs an explicit hand-off from
// the last producer to the selection).  Workgroup b computes the logits of
// expert rows NT/256 * b .. (one row per 256 threads, router_rows.h), makes
// them visible at device scope, and counts itself in `counter`; the
// workgroup that arrives last (the counter read G - 1) makes the others'
// logits visible to itself, routes and buckets the whole batch exactly as
// route_bucket_small_kernel does, and sets the counter back to 0 for the
// next call.  No workgroup waits for another, so there is no forward-progress
// question: whichever workgroup is last finds every logit written.
template <int NCH, int V, int KC, int NT>
__global__ __launch_bounds__(NT) void router_route_bucket_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router, const float* __restrict__ bias, int T,
    int H, int E, int k, float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos, int32_t* __restrict__ counter) {
  constexpr int kRows = NT / kRtThreads;                     // expert rows per workgroup
  __shared__ double s_part[kRows][kRtWaves][kRsGroup];
  __shared__ int s_last;
  const int grp = threadIdx.x / kRtThreads;
  router_row<NCH>(x, w_router, T, H, E, logits, (int)blockIdx.x * kRows + grp, (int)threadIdx.x % kRtThreads,
                  s_part[grp]);
  // Hand-off.  Every wave waits until its logit stores have reached the
  // L2; after the barrier one thread counts the workgroup in with an
  // agent-scope acquire-release atomic: its release writes this XCD's L2 back
  // (every store of the workgroup is in it by then), its acquire invalidates
  // this CU's L1 and this XCD's L2, so the workgroup that arrives last reads
  // every other's logits from memory.  One fence pair per workgroup: a
  // device-scope fence in every wave costs an L2 write-back and invalidate
  // per wave.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  route_bucket_block<V, KC, NT>(logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset,
                                active_experts, n_active, route_src, route_pos);
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int id_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

moe_status check_route_args(const float* logits, const float* bias, int T, int E, int k, const int32_t* topk_idx,
                            const float* topk_w) {
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL_POINTER;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w) || (bias && !aligned16(bias)))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_bucket_args(int T, int E, int k, const int32_t* a, const int32_t* b, const int32_t* c,
                             const int32_t* d, const int32_t* e, const int32_t* f) {
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_SHAPE;
  const long long R = (long long)T * k;
  if (E > 1024 || R > (1ll << 24)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!a || !b || !c || !d || !e || !f) return MOE_ERR_NULL_POINTER;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d) || !aligned16(e) || !aligned16(f))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

void launch_route(const float* logits, const float* bias, int T, int E, int k, int32_t* topk_idx, float* topk_w,
                  hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  const int V = (E + kWave - 1) / kWave;
#define MOE_RT(VV)                                                                                  \
  if (k == kUnrolledK) route_topk_kernel<VV, kUnrolledK><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w); \
  else route_topk_kernel<VV, 0><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w)
  if (V <= 1) { MOE_RT(1); }
  else if (V <= 2) { MOE_RT(2); }
  else if (V <= 4) { MOE_RT(4); }
  else if (V <= 8) { MOE_RT(8); }
  else { MOE_RT(16); }
#undef MOE_RT
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_topk(const float* logits, const float* bias, int T, int E, int k,
                                     int32_t* topk_idx, float* topk_w, void* stream) {
  using namespace moe;
  const moe_status st = check_route_args(logits, bias, T, E, k, topk_idx, topk_w);
  if (st != MOE_OK || T == 0) return st;
  launch_route(logits, bias, T, E, k, topk_idx, topk_w, static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" moe_status moe_bucket_routes(const int32_t* topk_idx, int T, int E, int k,
                                        int32_t* expert_count, int32_t* expert_offset,
                                        int32_t* active_experts, int32_t* n_active,
                                        int32_t* route_src, int32_t* route_pos, void* stream) {
  using namespace moe;
  const moe_status st = check_bucket_args(T, E, k, expert_count, expert_offset, active_experts, n_active,
                                          route_src, route_pos);
  if (st != MOE_OK || T == 0) return st;
  if (!topk_idx) return MOE_ERR_NULL_POINTER;
  if (!aligned16(topk_idx)) return MOE_ERR_MISALIGNED;
  bucket_routes_kernel<<<1, kBucketThreads, 0, static_cast<hipStream_t>(stream)>>>(
      topk_idx, T * k, E, expert_count, expert_offset, active_experts, n_active, route_src,
      route_pos, WorkLists{});
  return launch_status();
}

namespace moe {

moe_status route_bucket(const float* logits, const float* bias, int T, int E, int k, int32_t* topk_idx,
                        float* topk_w, int32_t* expert_count, int32_t* expert_offset, int32_t* active_experts,
                        int32_t* n_active, int32_t* route_src, int32_t* route_pos, int32_t* scratch,
                        size_t scratch_bytes, hipStream_t s, const WorkLists* wl, bool* lists_built,
                        const SharedRows* sr, bool* sr_done) {
  if (lists_built) *lists_built = false;
  if (sr_done) *sr_done = false;
  const WorkLists lists = wl ? *wl : WorkLists{};
  moe_status st = check_route_args(logits, bias, T, E, k, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  st = check_bucket_args(T, E, k, expert_count, expert_offset, active_experts, n_active, route_src, route_pos);
  if (st != MOE_OK || T == 0) return st;
  const int bits = id_bits_for(E);
  const int V = (E + kWave - 1) / kWave;
  if (T <= kSmallMaxTokens && T * k <= kSmallMaxRoutes && E <= kSmallMaxExperts) {
    const SharedRows side = sr && sr->gu_nc > 0 ? *sr : SharedRows{};
    const int side_rows = side.gu_nc > 0 ? side.Is : 0;
    if (sr_done) *sr_done = side_rows > 0;
#define MOE_RBS1(VV, KK)                                                                                       \
  if (E <= 512 && T <= 8) route_bucket_small_kernel<VV, KK, 512><<<1 + (side_rows + kSmallSideWaves<512> - 1) / kSmallSideWaves<512>, 512, 0, s>>>(     \
      logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts, n_active, route_src, \
      route_pos, side); else                                                                                   \
  route_bucket_small_kernel<VV, KK, 1024><<<1 + (side_rows + kSmallSideWaves<1024> - 1) / kSmallSideWaves<1024>, 1024, 0, s>>>(                         \
      logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts, n_active, route_src, \
      route_pos, side)
#define MOE_RBS(VV) \
  if (k == kUnrolledK) MOE_RBS1(VV, kUnrolledK); else MOE_RBS1(VV, 0)
    if (V <= 1) { MOE_RBS(1); }
    else if (V <= 2) { MOE_RBS(2); }
    else if (V <= 4) { MOE_RBS(4); }
    else { MOE_RBS(8); }
#undef MOE_RBS
#undef MOE_RBS1
    return launch_status();
  }
  launch_route(logits, bias, T, E, k, topk_idx, topk_w, s);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const long long R = (long long)T * k;
  const long long C = (R + kBucketThreads - 1) / kBucketThreads;
  if (C > 1 && R <= kChunkedMaxRoutes) {
    bucket_chunked_kernel<<<(unsigned)C, kBucketThreads, 0, s>>>(topk_idx, (int)R, E, bits, expert_count,
                                                                  expert_offset, active_experts, n_active, route_src,
                                                                  route_pos, lists);
    st = launch_status();
    if (lists_built) *lists_built = st == MOE_OK && wl != nullptr;
    return st;
  }
  if (scratch && C > kChunkMinChunks && (size_t)C * E * sizeof(int32_t) <= scratch_bytes) {
    bucket_count_kernel<<<(unsigned)C, kBucketThreads, 0, s>>>(topk_idx, (int)R, E, scratch);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    bucket_scan_kernel<<<1, kBucketThreads, 0, s>>>(scratch, (int)C, E, expert_count, expert_offset, active_experts,
                                                    n_active, lists);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    bucket_scatter_kernel<<<(unsigned)C, kBucketThreads, 0, s>>>(topk_idx, (int)R, E, bits, scratch, expert_offset,
                                                                 route_src, route_pos);
    st = launch_status();
    if (lists_built) *lists_built = st == MOE_OK && wl != nullptr;
    return st;
  }
  bucket_routes_kernel<<<1, kBucketThreads, 0, s>>>(topk_idx, (int)R, E, expert_count, expert_offset,
                                                     active_experts, n_active, route_src, route_pos, lists);
  st = launch_status();
  if (lists_built) *lists_built = st == MOE_OK && wl != nullptr;
  return st;
}

}  // namespace moe

extern "C" moe_status moe_route_bucket(const float* logits, const float* bias, int T, int E, int k,
                                       int32_t* topk_idx, float* topk_w,
                                       int32_t* expert_count, int32_t* expert_offset,
                                       int32_t* active_experts, int32_t* n_active,
                                       int32_t* route_src, int32_t* route_pos, void* stream) {
  return moe::route_bucket(logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts,
                           n_active, route_src, route_pos, nullptr, 0, static_cast<hipStream_t>(stream));
}

extern "C" moe_status moe_router_route_bucket(const uint16_t* x, const float* w_router, const float* bias, int T,
                                              int H, int E, int k, float* logits, int32_t* topk_idx, float* topk_w,
                                              int32_t* expert_count, int32_t* expert_offset,
                                              int32_t* active_experts, int32_t* n_active, int32_t* route_src,
                                              int32_t* route_pos, int32_t* counter, void* stream) {
  using namespace moe;
  if (T < 0 || E < 1 || H < 8 || H % 8 != 0) return MOE_ERR_INVALID_SHAPE;
  moe_status st = check_route_args(logits, bias, T, E, k, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  st = check_bucket_args(T, E, k, expert_count, expert_offset, active_experts, n_active, route_src, route_pos);
  if (st != MOE_OK) return st;
  if (H > kRtMaxH || ((long long)T + 63) / 64 > 65535) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !counter) return MOE_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(counter)) return MOE_ERR_MISALIGNED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T > kSmallMaxTokens || T * k > kSmallMaxRoutes || E > kSmallMaxExperts) {
    // larger batches and more than 512 experts: the projection, then the
    // routing, as two calls
    st = moe_router_logits(x, w_router, T, H, E, logits, stream);
    if (st != MOE_OK) return st;
    return route_bucket(logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts,
                        n_active, route_src, route_pos, nullptr, 0, s);
  }
  const int V = (E + kWave - 1) / kWave;
  const int nch = (H / 8 + kRtThreads - 1) / kRtThreads;     // 16-byte pieces per thread: 1 or 2
  // 1024 threads: four expert rows per workgroup (E / 4 workgroups count in;
  // measured faster than two rows per 512-thread workgroup, whose 2x more
  // hand-offs cost more than the smaller workgroup saves in the selection,
  // and than eight or more rows per workgroup, which slows the projection)
  constexpr int kNt = 1024;
  const unsigned grid = (unsigned)((E + kNt / kRtThreads - 1) / (kNt / kRtThreads));
#define MOE_RRB1(VV, KK)                                                                                      \
  if (nch <= 1) router_route_bucket_kernel<1, VV, KK, kNt><<<grid, kNt, 0, s>>>(x, w_router, bias, T, H, E, k, \
      logits, topk_idx, topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos,    \
      counter); else                                                                                          \
  router_route_bucket_kernel<2, VV, KK, kNt><<<grid, kNt, 0, s>>>(x, w_router, bias, T, H, E, k, logits,       \
      topk_idx, topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, counter)
#define MOE_RRB(VV) \
  if (k == kUnrolledK) MOE_RRB1(VV, kUnrolledK); else MOE_RRB1(VV, 0)
  if (V <= 1) { MOE_RRB(1); }
  else if (V <= 2) { MOE_RRB(2); }
  else if (V <= 4) { MOE_RRB(4); }
  else { MOE_RRB(8); }
#undef MOE_RRB
#undef MOE_RRB1
  return launch_status();
}
