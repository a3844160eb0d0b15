// moe_expert_ffn: routed NVFP4 SwiGLU experts with a weighted, fixed-order unroute.
//
// The chain of the SM70 design note (page "Persistent execution for Flash-Next
// GGUF on SM70", sections "What the measurements establish" and "First
// implementation boundary"): gate/up fused with SiLU * multiply, then down,
// then the weighted unroute with routes summed in a fixed order rather than
// by arrival-ordered floating-point atomics.  Unique-expert reuse: a task owns
// (active expert, row tile) and streams those weight rows from HBM once for
// all of the expert's routes (the note's first boundary, step 2; the b12x
// kernel's cost is the weight bytes of the unique experts - page "Qwen3.8
// Flash Next on LiL/vLLM: why the MTP decode step is host-bound, and what
// LMCache does and does not do to it", section "11.13 Where the decode
// step's time actually goes").
//
// Kernels on one stream; the kernel boundaries order the phases, so no
// workgroup ever waits for another (small batches replace the last two with
// down_combine_kernel):
//   gate_up_kernel  task (active slot a, tile of I rows): h[p, rows] =
//                   bf16(SiLU(Wg x) * (Wu x)) for every route p of the expert
//   down_kernel     task (active slot a, tile of H rows): o[p, rows] = Wd h[p]
//   combine_kernel  y[t] = bf16( sum_{j=0}^{k-1} w[t,j] * o[route_pos[t*k+j]] ),
//                   j in slot order
// h and o live in the caller's workspace, indexed by bucket position p.  For
// small batches (all routes' h fit in 64 KB of LDS) down_combine_kernel does
// the down projection and the unroute in one pass split by output rows.
//
// Row tiles (gfx950).  A wavefront reads whole rows: Lr lanes share a row and
// each lane reads one 16-byte chunk of e2m1 codes (32 values) plus its two
// e4m3 scales, with buffer loads from a per-expert resource.  The whole byte
// offset goes in the instruction's vector offset, which the hardware range
// check covers (the scalar offset is added after the check): rows past the
// matrix read as zero, so ragged tiles need no predication and no index can
// fault.  Byte pairs become bf16 with
// v_cvt_scalef32_pk_bf16_fp4 (exact at scale 1), v_dot2 multiplies them
// pairwise with the bf16 operand (x or h) and accumulates in fp32, one scale
// multiplies each 16-value block, and the partial sums of a row are added
// across its lanes with DPP row operations and v_permlane{16,32}_swap in a
// fixed order.  A tile's weight rows are loaded once and stay in registers
// while the expert's routes are processed one at a time, which keeps the
// kernels at 4+ waves per SIMD - the VALU needs that many waves to reach its
// issue rate.
//
// Issue order.  Vector loads complete in order (one counter per wave), so a
// load issued after a tile's weight rows cannot be used before all of them
// have arrived.  Each kernel therefore issues everything its first use needs
// before the weight stream (scale tiles, operand rows) or fetches it through
// the scalar path (routing metadata: s_load, its own counter), and a WG's
// dependent round trips all happen while its weights are in flight.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "row_dot.h"
#include "select.h"
#include "shared_rows.h"
#include "work_list.h"

namespace moe {
namespace {

struct FfnParams {
  const uint16_t* x;
  const uint8_t* wg;
  const uint8_t* sg;
  const uint8_t* wu;
  const uint8_t* su;
  const uint8_t* wd;
  const uint8_t* sd;
  const float* gsc;
  const float* topk_w;
  const int32_t* topk_idx;   // route-slot mode of the small-batch down/unroute (else unused)
  const int32_t* count;
  const int32_t* offset;
  const int32_t* active;
  const int32_t* n_active_ptr;
  const int32_t* route_src;
  const int32_t* route_pos;
  int T, H, I, E, k;
  uint16_t* h;   // workspace: [R, I] bf16, row = bucket position
  uint16_t* o;   // workspace: [R, H] fp16 bits, row = bucket position
  uint16_t* y;
  int lr_gu;     // lanes per gate/up row (power of two, <= 64)
  int lr_d;      // lanes per down row
  int mfma_min;  // experts with at least this many routes take the MFMA kernels (0: none do)
  const uint8_t* packed;   // the weights also in MFMA tile order (moe_pack_weights), or null
  int32_t* plan;           // workspace: the gate/up MFMA kernels' items (plan_kernel, see there)
  int32_t* plan_down;      // workspace: the down MFMA kernels' items (chunks of up to 128 routes)
  int plan_max;            // capacity of the item list
  int32_t* rd_list;        // workspace: row-dot experts, most routes first (plan_kernel)
  int rd_plan;             // the row-dot kernels take their experts from rd_list
  int32_t* queues;         // workspace: unit counters of the streaming down kernel
  SharedRows sr;           // shared-expert down rows riding along in gate_up_kernel (dn_nc 0: none)
  int layer_items;         // MFMA gate/up: items per XCD that fill its CUs once (0: list order)
  int split_items;         // work lists: items of at most 64 routes up to this many (WorkLists)
};

constexpr int kGuUnits = 4;          // gate rows (and as many up rows) per wave per tile
constexpr int kDUnits = 8;           // down rows per lane group per tile
// Scale bytes of one tile: rows_per_tile * cols/16 = 4 waves * (64/Lr) rows *
// units * 2*Lr bytes = 512 * units bytes when each lane reads one chunk.
constexpr int kScaleTileBytes = 2048;

// Routing metadata is read through the scalar memory path (s_load): it is
// wave-uniform, and scalar loads are counted apart from the vector loads, so
// a metadata fetch issued while a tile's weight rows are in flight does not
// have to wait for them (vector loads complete in order).
typedef const __attribute__((address_space(4))) int32_t* scalar_ptr;
typedef const __attribute__((address_space(4))) float* scalar_fptr;
__device__ __forceinline__ int sload(const int32_t* base, int i) { return ((scalar_ptr)base)[i]; }
__device__ __forceinline__ float sload(const float* base, int i) { return ((scalar_fptr)base)[i]; }

// Expert id of active slot a (-1 past the active list), clamped into range:
// inputs that violate the bucket precondition give wrong results but no
// out-of-bounds access.
__device__ __forceinline__ int slot_expert(const FfnParams& p, int a) {
  const int e = sload(p.active, a);
  return e < 0 ? -1 : min(e, p.E - 1);
}

// First bucket position and route count of expert e, clamped into [0, R].
__device__ __forceinline__ void expert_routes(const FfnParams& p, int e, int& off, int& cnt) {
  const int R = p.T * p.k;
  off = min(max(sload(p.offset, e), 0), R);
  cnt = min(max(sload(p.count, e), 0), R - off);
}

// True when expert e's routes go to the MFMA kernels instead (decided before
// any weight load is issued, so the two paths never both stream an expert).
__device__ __forceinline__ bool takes_mfma(const FfnParams& p, int e) {
  if (p.mfma_min <= 0) return false;
  int off, cnt;
  expert_routes(p, e, off, cnt);
  return cnt >= p.mfma_min;
}

// Expert of the a-th row-dot workgroup group, or -1 when there is none.
// With the plan (batches above 16 tokens) the experts come most routes first
// (rd_list[0] = their count, then the list), so the longest workgroups start
// first; otherwise in active-slot order, skipping the experts the MFMA
// kernels take.
__device__ __forceinline__ int row_dot_expert(const FfnParams& p, int a) {
  if (p.rd_plan) {
    const int n = sload(p.rd_list, 0), e = sload(p.rd_list, 1 + a);   // a < min(E, T*k): in the list
    return a < n ? min(max(e, 0), p.E - 1) : -1;
  }
  const int e = slot_expert(p, a);
  return (e < 0 || takes_mfma(p, e)) ? -1 : e;
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void wait_vector_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------ gate/up

// Activation rows staged per group of routes (16 KB of LDS).
constexpr int kXStageBytes = 16384;
// 16-byte activation pieces per thread when every token's row is staged up front.
constexpr int kXLoads = kXStageBytes / 16 / kThreads;

// Gate and up rows of one I tile for all routes of expert e.  Each wave holds
// kGuUnits gate rows and the same up rows; with 64 lanes per row the four
// units' sums are scattered so that lane row r ends with unit r.
//
// Issue order.  Small batches (every token's activation row fits the 16 KB
// stage): all activation rows (into registers: they do not depend on the
// routing), the tile's scale bytes (2 KB gate + 2 KB up, one 16-byte load
// per thread), then the weight rows, unit by unit; the expert's route range
// and first token come through the scalar path while the rows are in
// flight.  Activations and scales go to LDS as soon as they land, and each
// unit's products start as soon as its rows arrive, so only the last unit's
// work is left when the stream ends.  Larger batches: scale bytes, weight
// rows, then the activation rows of each group of routes straight into LDS
// once the route range is known; all of them land before any product.
template <int LG>
__device__ __forceinline__ void gate_up_tile(const FfnParams& p, const Geo<LG, kGuUnits>& g, uint8_t* s_sc,
                                             uint8_t* s_x, int e, int tile) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const uint32_t code_row = (uint32_t)p.H / 2, scale_row = (uint32_t)p.H / 16;
  const uint32_t mat_codes = (uint32_t)p.I * code_row, mat_scales = (uint32_t)p.I * scale_row;
  const uint32_t blk = (uint32_t)g.rpt * scale_row;            // 2048 bytes
  const int row_bytes = p.H * 2;
  const int group = max(1, min(kXStageBytes / row_bytes, 64));   // x rows in the LDS stage (<= 16 KB)
  const uint32_t x_bytes = (uint32_t)p.T * (uint32_t)row_bytes;
  // small batches: every token's activation row is staged before the weights
  const bool x_first = p.T <= group;
  u32x4 xv[kXLoads];
  if (x_first) {
    const auto rx = make_rsrc(p.x, x_bytes);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + i * kThreads) * 16, 0, 0);
  }
  compiler_fence();
  const int half = (int)(g.wave >= kWavesPerBlock / 2);          // wave-uniform: waves 2, 3 load up scales
  const uint32_t sbyte = (uint32_t)(tid & (kThreads / 2 - 1)) * 16;
  const auto rs = make_rsrc((half ? p.su : p.sg) + (size_t)e * mat_scales, mat_scales);
  const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rs, sbyte + (uint32_t)tile * blk, 0, kStreamAux);
  compiler_fence();
  const auto rg = make_rsrc(p.wg + (size_t)e * mat_codes, mat_codes);
  const auto ru = make_rsrc(p.wu + (size_t)e * mat_codes, mat_codes);
  const uint32_t lane_c = (uint32_t)g.sub * code_row + (uint32_t)g.sl * 16;
  uint4 cg[kGuUnits], cu[kGuUnits];
#pragma unroll
  for (int u = 0; u < kGuUnits; ++u) {
    const uint32_t r0 = (uint32_t)g.row0(tile, u);
    cg[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rg, lane_c + r0 * code_row, 0, kStreamAux));
    cu[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(ru, lane_c + r0 * code_row, 0, kStreamAux));
  }
  compiler_fence();
  int off, cnt;
  expert_routes(p, e, off, cnt);
  const float Gg = sload(p.gsc, e * 3 + 0), Gu = sload(p.gsc, e * 3 + 1);
  auto token_of = [&](int pos) { return min(max(sload(p.route_src, pos) / p.k, 0), p.T - 1); };

  // h[pos, rows of this tile] for one route whose x row sits at s_x + xs*row_bytes.
  // Each unit's weight rows are touched just before their own products, so
  // on the first route the compiler waits for unit u's loads only.
  auto route = [&](int pos, int xs) {
    const float one = opaque_one();
    uint32_t xr[16];
    load_operand_chunk(reinterpret_cast<const uint16_t*>(s_x + (size_t)xs * row_bytes), g.sl, xr);
    float ag[kGuUnits], au[kGuUnits];
#pragma unroll
    for (int u = 0; u < kGuUnits; ++u) {
      const int rin = (u * kWavesPerBlock + g.wave) * g.rpw + g.sub;   // row within the tile
      const uint32_t sg = *reinterpret_cast<const uint16_t*>(s_sc + rin * scale_row + g.sl * 2);
      const uint32_t su = *reinterpret_cast<const uint16_t*>(s_sc + blk + rin * scale_row + g.sl * 2);
      ag[u] = dot_chunk(cg[u], sg, xr, 0.0f, one);
      au[u] = dot_chunk(cu[u], su, xr, 0.0f, one);
    }
    if constexpr (LG == 64) {
      static_assert(kGuUnits == 4, "the row scatter maps 4 units to 4 lane rows");
      const int row = g.row0(tile, lane >> 4);
      const float gs = rows_scatter4(row16_sum(ag[0]), row16_sum(ag[1]), row16_sum(ag[2]), row16_sum(ag[3])) * Gg;
      const float us = rows_scatter4(row16_sum(au[0]), row16_sum(au[1]), row16_sum(au[2]), row16_sum(au[3])) * Gu;
      if ((lane & 15) == 0 && row < p.I) p.h[(size_t)pos * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
    } else {
#pragma unroll
      for (int u = 0; u < kGuUnits; ++u) {
        const int row = g.row0(tile, u) + g.sub;
        const float gs = group_sum(ag[u], g.lr) * Gg;
        const float us = group_sum(au[u], g.lr) * Gu;
        if (g.sl == 0 && row < p.I) p.h[(size_t)pos * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
      }
    }
  };

  if (x_first) {
    // the first route's token comes through the scalar path while the rows
    // are in flight; x and the scale bytes go to LDS as soon as they land
    // (before the weight rows: the loads complete in order), and the waves
    // meet at a barrier that does not wait for the weight rows
    const int tok0 = cnt > 0 ? token_of(off) : 0;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const uint32_t q = (uint32_t)(tid + i * kThreads) * 16;
      if (q < x_bytes) *reinterpret_cast<u32x4*>(s_x + q) = xv[i];
    }
    *reinterpret_cast<u32x4*>(s_sc + half * blk + sbyte) = sv;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    // the first route outside any loop: its unit-by-unit waits stay per use
    // (before a loop the compiler would wait for every load)
    if (cnt > 0) route(off, tok0);
#pragma unroll 1
    for (int i = 1; i < cnt; ++i) route(off + i, token_of(off + i));
    return;
  }

  // larger batches: the activation rows of each group of routes go straight
  // into LDS once the route range is known
  const int pieces = row_bytes / 16;                             // 16-byte pieces of one x row
  for (int g0 = 0; g0 < cnt; g0 += group) {
    const int ng = min(group, cnt - g0);
    if (g0 > 0) __syncthreads();                                 // previous group's x reads done
    for (int i = 0; i < ng; ++i) {
      const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)token_of(off + g0 + i) * p.H);
      for (int q0 = g.wave * kWave; q0 < pieces; q0 += kThreads)
        if (q0 + lane < pieces)
          __builtin_amdgcn_global_load_lds(src + q0 + lane, s_x + (size_t)i * row_bytes + (size_t)q0 * 16, 16, 0, 0);
    }
    if (g0 == 0) {
      compiler_fence();
      *reinterpret_cast<u32x4*>(s_sc + half * blk + sbyte) = sv;
    }
    wait_vector_loads();
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < ng; ++i) route(off + g0 + i, i);
  }
}

template <int LG>
__global__ __launch_bounds__(kThreads, 4) void gate_up_kernel(FfnParams p, int n_tasks) {
  __shared__ __align__(16) uint8_t s_sc[2 * kScaleTileBytes];
  extern __shared__ __align__(16) uint8_t s_x[];                // activation rows of a group of routes
  const Geo<LG, kGuUnits> g(p.lr_gu, p.I);
  // one task per workgroup (the host launches n_tasks of them after the
  // shared rows' ones): no loop around the tile, so the compiler's load waits
  // stay per use
  // the first workgroups take the down rows of a shared expert
  // (moe_step_shared), if any: dispatched first, they run beside the tasks
  // instead of after them
  const int side = se_down_side_blocks(p.sr, kThreads / kWave);
  if ((int)blockIdx.x < side) {
    se_down_side(p.sr, (int)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6),
                 threadIdx.x & (kWave - 1));
    return;
  }
  const int task = blockIdx.x - side;
  if (task >= n_tasks) return;
  const int a = task / g.tiles, tile = task - a * g.tiles;
  const int e = row_dot_expert(p, a);
  if (e < 0) return;
  gate_up_tile<LG>(p, g, s_sc, s_x, e, tile);
}

// ------------------------------------------------------------------ selection + gate/up (small batches)

// A small batch's selection and gate/up in one launch, with no hand-off
// between workgroups: workgroup (r, tile), r = t*k + j, selects token t's
// j-th expert itself (its first wave runs the rounds of the selection up to
// round j; select.h, the rule of moe_route_topk, so the result is that
// call's bit for bit) and computes the gate/up rows of tile `tile` of that
// expert for that one route: h[r, rows] in the workspace, indexed by flat
// route id.  Every token's selection is repeated by k * tiles workgroups
// (one wave each; slot 0's start streaming after one round, slot k-1's after
// all k), and an expert picked by several
// tokens is streamed once per route: at four tokens the distinct experts
// carry ~96% of the route-issued bytes, and the weights start streaming
// without waiting for a routing kernel, its boundary and a dependent read of
// the active list.  Rows of H = 2048 (one 16-byte chunk per lane, 64 lanes
// per row), as gate_up_kernel<64>.  One more workgroup, the launch's last,
// writes every routing output (small_route_bucket): at 59 registers eight
// of these workgroups fit a CU, so it runs beside the others.
constexpr int kSgXBytes = 4096;           // one activation row of H = 2048
constexpr int kSgMaxRoutes = 40;          // routes of a small batch (the small step's limit)

// The routing outputs of a small batch (at most kSgMaxRoutes routes), by one
// workgroup of kThreads threads of the selection launch, beside the gate/up
// workgroups (which select for themselves and need none of it): wave w
// selects tokens w, w + 4, ... and writes topk_idx and topk_w; then the
// buckets - an LDS histogram of the route ids, one workgroup-wide scan of
// (routes, active experts) over four experts per thread for the offsets and
// active positions, and the stable scatter: route r goes to offset(e) plus
// the number of earlier routes to e (ballots per id bit; all routes lie in
// one wavefront), the route order of moe_bucket_routes.
template <int V, int KC>
__device__ __forceinline__ void small_route_bucket(const FfnParams& p, const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
  static_assert(kSgMaxRoutes <= kWave, "the scatter ranks one wavefront of routes");
  __shared__ int s_ids[kSgMaxRoutes];
  __shared__ int s_cnt[1024];                          // counts, then offsets
  __shared__ int s_wt[kWavesPerBlock];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int R = p.T * p.k;
#pragma unroll
  for (int i = 0; i < 4; ++i) s_cnt[4 * tid + i] = 0;
  for (int t = wave; t < p.T; t += kWavesPerBlock) {
    int e;
    float w;
    select_token<V, KC>(logits + (size_t)t * p.E, bias, p.E, p.k, lane, e, w);
    if (lane < p.k) {
      topk_idx[(size_t)t * p.k + lane] = e;
      topk_w[(size_t)t * p.k + lane] = w;
      s_ids[t * p.k + lane] = e;
    }
  }
  __syncthreads();
  if (tid < R) atomicAdd(&s_cnt[s_ids[tid]], 1);      // integer counts: order-free
  __syncthreads();
  int c[4], cs = 0, as = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = s_cnt[4 * tid + i];
    cs += c[i];
    as += c[i] > 0;
  }
  // exclusive scan over the workgroup of routes + (active experts << 16)
  const int v = cs + (as << 16);
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wt[wave] = inc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    base += w < wave ? s_wt[w] : 0;
    total += s_wt[w];
  }
  int scan = base + inc - v;
  const int total_active = total >> 16;
  int32_t* count = const_cast<int32_t*>(p.count);
  int32_t* offset = const_cast<int32_t*>(p.offset);
  int32_t* active = const_cast<int32_t*>(p.active);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    const int off = scan & 0xFFFF, apos = scan >> 16;
    if (e < p.E) {
      count[e] = c[i];
      offset[e] = off;
      if (c[i] > 0) active[apos] = e;
      if (e >= total_active) active[e] = -1;
    }
    s_cnt[e] = off;                                    // this thread's own entries: no barrier needed before
    scan += c[i] + ((c[i] > 0) << 16);
  }
  if (tid == 0) {
    offset[p.E] = total & 0xFFFF;
    *const_cast<int32_t*>(p.n_active_ptr) = total_active;
  }
  __syncthreads();
  if (wave == 0) {
    const bool valid = lane < R;
    const int e = valid ? s_ids[lane] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {                     // ids are below 1024
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    if (valid) {
      const int pos = s_cnt[e] + rank;
      const_cast<int32_t*>(p.route_src)[pos] = lane;
      const_cast<int32_t*>(p.route_pos)[lane] = pos;
    }
  }
}

template <int V, int KC>
__global__ __launch_bounds__(kThreads, 4) void select_gate_up_kernel(FfnParams p, const float* __restrict__ logits,
                                                                     const float* __restrict__ bias,
                                                                     int32_t* __restrict__ topk_idx,
                                                                     float* __restrict__ topk_w, int n_tasks) {
  __shared__ __align__(16) uint8_t s_sc[2 * kScaleTileBytes];
  __shared__ __align__(16) uint8_t s_x[kSgXBytes];
  __shared__ int s_e;
  const Geo<64, kGuUnits> g(64, p.I);
  // a shared expert's gate/up rows (one per wave) come first, so that their
  // loads are issued ahead of the tiles' weight stream
  const int se_blocks = p.sr.gu_nc > 0 ? (p.sr.Is + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  if ((int)blockIdx.x < se_blocks) {
    se_gate_up_side_small(p.sr, (int)blockIdx.x * kWavesPerBlock + g.wave, threadIdx.x & (kWave - 1));
    return;
  }
  const int task = (int)blockIdx.x - se_blocks;
  if (task >= n_tasks) {
    // the workgroup after the gate/up tiles: every routing output
    small_route_bucket<V, KC>(p, logits, bias, topk_idx, topk_w);
    return;
  }
  const int r = task / g.tiles, tile = task - r * g.tiles;
  const int t = r / p.k, j = r - t * p.k;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // token t's activation row, one 16-byte piece per thread: it does not
  // depend on the routing, so it is issued first
  const u32x4 xv =
      __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(p.x + (size_t)t * p.H, kSgXBytes), (uint32_t)tid * 16, 0, 0);
  compiler_fence();
  if (g.wave == (int)(blockIdx.x & (kWavesPerBlock - 1))) {
    // only slot j's expert: the rounds of the selection up to round j (the
    // routing workgroup writes the full top-k and its weights); the selecting
    // wave rotates with the workgroup so that neighbouring workgroups' rounds
    // run on different SIMDs
    const int e_j = select_slot<V, KC>(logits + (size_t)t * p.E, bias, p.E, j, lane);
    if (lane == 0) s_e = e_j;
  }
  *reinterpret_cast<u32x4*>(s_x + tid * 16) = xv;
  __syncthreads();
  const int e = min(max(__builtin_amdgcn_readfirstlane(s_e), 0), p.E - 1);

  // the tile of expert e, as gate_up_tile: scale bytes, then the weight rows
  const uint32_t code_row = (uint32_t)p.H / 2, scale_row = (uint32_t)p.H / 16;
  const uint32_t mat_codes = (uint32_t)p.I * code_row, mat_scales = (uint32_t)p.I * scale_row;
  const uint32_t blk = (uint32_t)g.rpt * scale_row;
  const int half = (int)(g.wave >= kWavesPerBlock / 2);
  const uint32_t sbyte = (uint32_t)(tid & (kThreads / 2 - 1)) * 16;
  const auto rs = make_rsrc((half ? p.su : p.sg) + (size_t)e * mat_scales, mat_scales);
  const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rs, sbyte + (uint32_t)tile * blk, 0, kStreamAux);
  compiler_fence();
  const auto rg = make_rsrc(p.wg + (size_t)e * mat_codes, mat_codes);
  const auto ru = make_rsrc(p.wu + (size_t)e * mat_codes, mat_codes);
  const uint32_t lane_c = (uint32_t)g.sub * code_row + (uint32_t)g.sl * 16;
  uint4 cg[kGuUnits], cu[kGuUnits];
#pragma unroll
  for (int u = 0; u < kGuUnits; ++u) {
    const uint32_t r0 = (uint32_t)g.row0(tile, u);
    cg[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rg, lane_c + r0 * code_row, 0, kStreamAux));
    cu[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(ru, lane_c + r0 * code_row, 0, kStreamAux));
  }
  compiler_fence();
  const float Gg = sload(p.gsc, e * 3 + 0), Gu = sload(p.gsc, e * 3 + 1);
  *reinterpret_cast<u32x4*>(s_sc + half * blk + sbyte) = sv;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  const float one = opaque_one();
  uint32_t xr[16];
  load_operand_chunk(reinterpret_cast<const uint16_t*>(s_x), g.sl, xr);
  float ag[kGuUnits], au[kGuUnits];
#pragma unroll
  for (int u = 0; u < kGuUnits; ++u) {
    const int rin = (u * kWavesPerBlock + g.wave) * g.rpw + g.sub;
    const uint32_t sg = *reinterpret_cast<const uint16_t*>(s_sc + rin * scale_row + g.sl * 2);
    const uint32_t su = *reinterpret_cast<const uint16_t*>(s_sc + blk + rin * scale_row + g.sl * 2);
    ag[u] = dot_chunk(cg[u], sg, xr, 0.0f, one);
    au[u] = dot_chunk(cu[u], su, xr, 0.0f, one);
  }
  static_assert(kGuUnits == 4, "the row scatter maps 4 units to 4 lane rows");
  const int row = g.row0(tile, lane >> 4);
  const float gs = rows_scatter4(row16_sum(ag[0]), row16_sum(ag[1]), row16_sum(ag[2]), row16_sum(ag[3])) * Gg;
  const float us = rows_scatter4(row16_sum(au[0]), row16_sum(au[1]), row16_sum(au[2]), row16_sum(au[3])) * Gu;
  if ((lane & 15) == 0 && row < p.I) p.h[(size_t)r * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
}

// ------------------------------------------------------------------ down

// Down rows of one H tile for all routes of expert e (weights loaded once).
// The tile's scale bytes (rpt rows of I/16 bytes, 4 KB) go to LDS with one
// 16-byte load per thread, issued before the weight rows; the expert's route
// range comes through the scalar path while the rows are in flight.
template <int LD>
__device__ __forceinline__ void down_tile(const FfnParams& p, const Geo<LD, kDUnits>& g, uint8_t* s_sc, int e,
                                          int tile) {
  const uint32_t code_row = (uint32_t)p.I / 2, scale_row = (uint32_t)p.I / 16;
  const uint32_t mat_codes = (uint32_t)p.H * code_row, mat_scales = (uint32_t)p.H * scale_row;
  const uint32_t blk = (uint32_t)g.rpt * scale_row;            // 4096 bytes
  const auto rs = make_rsrc(p.sd + (size_t)e * mat_scales, mat_scales);
  const u32x4 sv =
      __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)threadIdx.x * 16 + (uint32_t)tile * blk, 0, kStreamAux);
  compiler_fence();
  const auto rd = make_rsrc(p.wd + (size_t)e * mat_codes, mat_codes);
  const uint32_t lane_c = (uint32_t)g.sub * code_row + (uint32_t)g.sl * 16;
  uint4 cd[kDUnits];
#pragma unroll
  for (int u = 0; u < kDUnits; ++u) {
    const uint32_t r0 = (uint32_t)g.row0(tile, u);
    cd[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rd, lane_c + r0 * code_row, 0, kStreamAux));
  }
  compiler_fence();
  int off, cnt;
  expert_routes(p, e, off, cnt);
  *reinterpret_cast<u32x4*>(s_sc + threadIdx.x * 16) = sv;
  __syncthreads();
  uint32_t vd[kDUnits];
#pragma unroll
  for (int u = 0; u < kDUnits; ++u) {
    const int rin = (u * kWavesPerBlock + g.wave) * g.rpw + g.sub;
    vd[u] = *reinterpret_cast<const uint16_t*>(s_sc + rin * scale_row + g.sl * 2);
  }
  const float Gd = sload(p.gsc, e * 3 + 2);
  for (int t = 0; t < cnt; ++t) {
    const int pos = off + t;
    const float one = opaque_one();
    uint32_t hr[16];
    load_operand_chunk(p.h + (size_t)pos * p.I, g.sl, hr);
    float ad[kDUnits];
#pragma unroll
    for (int u = 0; u < kDUnits; ++u) ad[u] = dot_chunk(cd[u], vd[u], hr, 0.0f, one);
#pragma unroll
    for (int u = 0; u < kDUnits; ++u) {
      const int row = g.row0(tile, u) + g.sub;
      const float v = (LD == 16 ? row16_sum(ad[u]) : group_sum(ad[u], g.lr)) * Gd;
      // with 16 lanes per row, lane u of the row stores unit u
      if (g.sl == (LD == 16 ? u : 0) && row < p.H) p.o[(size_t)pos * p.H + row] = f32_to_f16_bits(v);
    }
  }
}

template <int LD>
__global__ __launch_bounds__(kThreads, 4) void down_kernel(FfnParams p, int n_tasks) {
  __shared__ __align__(16) uint8_t s_sc[2 * kScaleTileBytes];
  const Geo<LD, kDUnits> g(p.lr_d, p.H);
  const int task = blockIdx.x;                  // one task per workgroup
  if (task >= n_tasks) return;
  const int a = task / g.tiles, tile = task - a * g.tiles;
  const int e = row_dot_expert(p, a);
  if (e < 0) return;
  down_tile<LD>(p, g, s_sc, e, tile);
}

// ------------------------------------------------------------------ MFMA tiles (experts with many routes)

// For an expert with many routes the projections are dense contractions:
// gate/up is [I x H] x [H x routes] twice, down is [H x I] x [I x routes].
// A workgroup owns 128 weight rows of one expert (the same rows of W_gate
// and W_up for gate/up) and one chunk of up to 128 of its routes (one item
// of the work plan below: an expert with more routes has one workgroup per
// chunk, running side by side); each of its four waves owns 32 of the rows
// and all of the chunk's routes.  The packed down kernel gives each wave two
// 32-row tiles (256 rows per workgroup), so every B fragment read feeds two
// MFMAs.
//
// v_mfma_f32_32x32x16_bf16 with the weights as A (32 rows x 16) and the
// routes' operand rows as B (16 x 32 routes).  Lane layout (checked on the
// device): A lane l holds row l%32, reduction indices 8*(l/32)..+8; B lane l
// holds column l%32, the same indices; D register r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l%32.  The reduction index is permuted
// consistently in A and B: within a 64-wide step, instruction kk of lane
// half h covers k = 32h + 8kk .. +8, so a lane's four A fragments of a step
// are 32 consecutive weights of its row - one 16-byte load of e2m1 codes and
// the two e4m3 scales of those blocks, dequantised in registers to exact
// bf16 (e2m1 * e4m3 is exact in bf16; the fp32 global scale is applied to
// the accumulator).  Each weight is loaded and dequantised once.
//
// The operand rows (x gathered by token for gate/up, the expert's contiguous
// h rows for down) go straight into a four-stage LDS ring with
// global_load_lds, 16-byte chunks placed at chunk ^ ((row >> 1) & 7) so that
// the B-fragment reads of 16 lanes hit 16 different bank groups.  Weight
// codes and scales go into a four-entry register ring.  A step's loads are
// issued two steps ahead (measured: one and three steps ahead are no faster
// at prefill, and three is ~2 µs slower at 256 Zipf-routed tokens, whose
// loads then crowd the memory system for little cover).
// Workgroups are numbered so that the n-tiles of one expert share an XCD
// (workgroups are dealt round robin to the 8 XCDs): its gathered rows are
// then read from that XCD's L2 after the first tile.
//
// Epilogue: gate/up writes h = bf16(SiLU(g Gg) * (u Gu)); down writes
// o = fp16(Gd * acc) for the combine kernel.
constexpr int kMmThreads = 256;
constexpr int kMmRows = 128;                 // weight rows per workgroup (32 per wave)
constexpr int kMmRoutes = 128;               // routes per chunk
constexpr int kMmK = 64;                     // reduction per step
constexpr int kMmStages = 4;                 // operand-ring stages
constexpr int kMmLead = 2;                   // one-unit kernel: steps issued ahead of the one in use
constexpr int kMmStageBytes = kMmRoutes * kMmK * 2;   // 16 KB of operand rows per step
constexpr int kXcds = 8;
static_assert(kMmRows == kPackRows && kMmK == kPackK, "packed weights follow the MFMA tile");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// e2m1 code pair `B` of `word` times `scale`, as two bf16 (exact).
template <int B>
__device__ __forceinline__ uint32_t fp4x2_scaled(uint32_t word, float scale) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, B);
  return pack_bf16x2(v.x * scale, v.y * scale);
}

// 32 weights (16 code bytes, two block-scale bytes) -> four A fragments of 8 bf16.
__device__ __forceinline__ void dequant_frags(const uint4 codes, uint32_t s2, bf16x8 (&fr)[4]) {
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)s2, 1);
  const uint32_t c[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sc = q < 2 ? s0 : s1;
    const uint4 v = make_uint4(fp4x2_scaled<0>(c[q], sc), fp4x2_scaled<1>(c[q], sc), fp4x2_scaled<2>(c[q], sc),
                               fp4x2_scaled<3>(c[q], sc));
    fr[q] = __builtin_bit_cast(bf16x8, v);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence.  __syncthreads() adds a
// workgroup-scope fence, which waits for every outstanding vector load -
// including the prefetched steps.  Inside the step loop the only data other
// waves read is operand rows written to LDS by buffer_load ... lds, whose
// completion each wave establishes with wait_vm before the barrier.
__device__ __forceinline__ void step_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// The barrier after which a stage is refilled: each wave first waits for its
// own LDS reads of that stage to return.  The MFMAs that consume them may be
// scheduled after the barrier, and a read still queued in the LDS unit could
// otherwise see rows that another wave's next buffer_load ... lds has
// already written.
__device__ __forceinline__ void stage_release_barrier() {
  compiler_fence();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// NSUB: row tiles of W_down per wave (down only; gate/up always has two A
// operands, the same rows of W_gate and W_up).  Two row tiles per wave halve
// the workgroups of an expert, so each of its h rows is staged half as often
// and each B fragment read from LDS feeds two MFMAs.
template <bool GU, bool PACKED, int NSUB>
struct MmTile {
  static constexpr int NA = GU ? 2 : NSUB;             // A operands per wave
  static constexpr int kLoadsPerStep = 4 + 2 * NA;     // per thread: 4 operand chunks, codes + scales per operand
  uint8_t* s_x[kMmStages];                             // one LDS array per stage
  __amdgpu_buffer_rsrc_t rc[NA], rs[NA], rb;
  uint32_t w_voff[NA], s_voff[NA];                     // this lane's slice of each A operand (packed: from its tile)
  uint32_t x_goff[4];                                  // operand chunk sources, per step add ks*128
  int wave, lane;
  uint4 wc[kMmStages][NA];
  // the scale pairs stay 16-bit until their step uses them: widened in the
  // ring, the compiler zero-extends the ones still in flight at the loop's
  // back edge and waits for their loads there, draining the prefetch
  uint16_t wsv[kMmStages][NA];

  template <int T>
  __device__ __forceinline__ void issue(int ks) {
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      if constexpr (PACKED) {
        // one contiguous kilobyte of codes (and 128 bytes of scales) per wave,
        // read once; the tile offset is in the range-checked vector offset
        wc[T][m] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rc[m], w_voff[m], (uint32_t)ks * 4096u, kStreamAux));
        wsv[T][m] = __builtin_amdgcn_raw_buffer_load_b16(rs[m], s_voff[m], (uint32_t)ks * 512u, kStreamAux);
      } else {
        // default cache policy: each load uses 32 of a row's 128 cached bytes,
        // the next three K steps use the rest
        wc[T][m] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rc[m], w_voff[m], (uint32_t)ks * (kMmK / 2), 0));
        wsv[T][m] = __builtin_amdgcn_raw_buffer_load_b16(rs[m], s_voff[m], (uint32_t)ks * (kMmK / 16), 0);
      }
    }
    uint8_t* stage = s_x[T];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, stage + (i * 4 + wave) * 1024, 16, x_goff[i], (uint32_t)ks * (kMmK * 2),
                                               0, 0);
  }
};

// Item order per XCD.  Workgroups reach an XCD's compute units in index
// order, one per CU first (a layer of L = CUs / row tiles items), then a
// second one beside the first ones.  When an XCD has between L and 2L items
// (one round, some CUs shared), item slot s of the second layer shares the
// CUs of slot s - L of the first, and the first-layer slots D .. L - 1 (D =
// items - L) keep their CUs to themselves.  Those slots take the L - D
// longest items (the list runs longest first), so that no long item shares its CUs
// with another: a CU running two workgroups gives each about half its issue
// slots, and a long item's partner set the launch's span at 256
// Zipf-routed tokens.  Returns the list rank of item slot s on XCD xcd; a
// bijection on 0 .. items-1, so the items computed do not change.
__device__ __forceinline__ int mfma_item_rank(int s, int xcd, int n_items, int L) {
  if (L <= 0) return s;
  const int items = (n_items - xcd + kXcds - 1) / kXcds;   // items of this XCD
  if (items <= L || items > 2 * L) return s;
  const int D = items - L;
  if (s < D) return s + (L - D);       // first layer, shared with a second-layer slot
  if (s < L) return s - D;             // first layer, alone: the longest items
  return s;                            // second layer
}

template <bool GU, bool PACKED, int NSUB>
__global__ __launch_bounds__(kMmThreads, 2) void ffn_mfma_kernel(FfnParams p) {
  static_assert(GU ? NSUB == 1 : (NSUB == 1 || PACKED), "several row tiles per wave: down on packed weights");
  using Tile = MmTile<GU, PACKED, NSUB>;
  constexpr int NMAT = Tile::NA;
  constexpr int kWgRows = kMmRows * (GU ? 1 : NSUB);          // weight rows per workgroup
  constexpr int LPS = Tile::kLoadsPerStep;
  // separate arrays per stage, so that reads of one stage are seen not to
  // alias the buffer_load ... lds writes in flight to the others
  __shared__ __align__(16) uint8_t s_x0[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x1[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x2[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x3[kMmStageBytes];
  __shared__ int s_row[kMmRoutes];                           // operand row per route of the chunk
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int N = GU ? p.I : p.H;                              // weight rows
  const int K = GU ? p.H : p.I;                              // reduction length
  const int tiles_n = (N + kWgRows - 1) / kWgRows;
  // workgroup b: XCD b % 8, j = b / 8, item (j / tiles_n) * 8 + XCD, n-tile
  // j % tiles_n: the tiles of one item share an XCD, and the items (longest
  // first) start in plan order
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  // the item is read together with the count (the list has room for every
  // item index of the grid), so the head costs one round of scalar loads
  const int32_t* const plan = GU ? p.plan : p.plan_down;
  const int n_items = min(sload(plan, 0), p.plan_max);
  const int it = mfma_item_rank(j / tiles_n, xcd, n_items, GU ? p.layer_items : 0) * kXcds + xcd;
  const int n0 = (j % tiles_n) * kWgRows;
  const int R = p.T * p.k;
  const int e = min(max(sload(plan, 4 + 4 * it), 0), p.E - 1);
  const int off = min(max(sload(plan, 5 + 4 * it), 0), R);
  const int cnt = min(max(sload(plan, 6 + 4 * it), 0), min(kMmRoutes, R - off));
  if (it >= n_items || cnt <= 0) return;

  Tile t;
  t.s_x[0] = s_x0;
  t.s_x[1] = s_x1;
  t.s_x[2] = s_x2;
  t.s_x[3] = s_x3;
  t.wave = wave;
  t.lane = lane;
  const uint32_t code_row = (uint32_t)K / 2, scale_row = (uint32_t)K / 16;
  const uint32_t mat_codes = (uint32_t)N * code_row, mat_scales = (uint32_t)N * scale_row;
  // operand rows: gate/up gathers x rows by token (the host keeps T*H*2 below
  // 2^31); down reads the item's own h rows, from a resource based at its
  // first route, so offsets stay below 128 rows whatever the batch size
  t.rb = GU ? make_rsrc(p.x, (uint32_t)p.T * (uint32_t)p.H * 2u)
            : make_rsrc(p.h + (size_t)off * p.I, (uint32_t)cnt * (uint32_t)p.I * 2u);
  const int steps = K / kMmK;
  if constexpr (PACKED) {
    // packed matrices: gate and up of every expert, then down (tile order)
    const size_t gu_mat = packed_matrix_bytes(p.I, p.H);
    const size_t mat = packed_matrix_bytes(N, K), codes = packed_code_bytes(N, K);
    const uint8_t* base[2] = {p.packed + (GU ? 0 : 2 * (size_t)p.E * gu_mat), p.packed + (size_t)p.E * gu_mat};
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const uint8_t* me = base[GU ? m : 0] + (size_t)e * mat;
      t.rc[m] = make_rsrc(me, (uint32_t)codes);
      t.rs[m] = make_rsrc(me + codes, (uint32_t)(mat - codes));
      // gate/up: both operands from the workgroup's tile; down: tile m of it
      const uint32_t tile_step0 = (uint32_t)(n0 / kMmRows + (GU ? 0 : m)) * (uint32_t)steps;
      t.w_voff[m] = (uint32_t)(wave * 64 + lane) * 16 + tile_step0 * 4096u;
      t.s_voff[m] = (uint32_t)(wave * 64 + lane) * 2 + tile_step0 * 512u;
    }
  } else {
    const uint8_t* wbase[2] = {GU ? p.wg : p.wd, p.wu};
    const uint8_t* sbase[2] = {GU ? p.sg : p.sd, p.su};
    const int wrow = n0 + wave * 32 + l32;                   // this lane's weight row
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      t.rc[m] = make_rsrc(wbase[m] + (size_t)e * mat_codes, mat_codes);
      t.rs[m] = make_rsrc(sbase[m] + (size_t)e * mat_scales, mat_scales);
      t.w_voff[m] = (uint32_t)wrow * code_row + (uint32_t)half * 16;
      t.s_voff[m] = (uint32_t)wrow * scale_row + (uint32_t)half * 2;
    }
  }

  {
    // one chunk of at most kMmRoutes routes: bucket positions off .. off + cnt - 1
    const int m0 = 0, mc = cnt;
    const int mtiles = (mc + 31) >> 5;
    __syncthreads();                                         // previous chunk done with LDS
    if (tid < kMmRoutes) {
      const int loc = m0 + min(tid, mc - 1);                 // rows past the chunk repeat its last route
      s_row[tid] = GU ? min(max(p.route_src[off + loc] / p.k, 0), p.T - 1) : loc;
    }
    __syncthreads();
    // operand chunk q = (4i + wave)*64 + lane sits at row q/8, position q%8,
    // and holds source chunk (q%8) ^ ((row >> 1) & 7) of that row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = (i * 4 + wave) * 64 + lane;
      const int row = q >> 3, c = (q & 7) ^ ((row >> 1) & 7);
      t.x_goff[i] = (uint32_t)s_row[row] * (uint32_t)K * 2u + (uint32_t)c * 16;
    }
    f32x16 acc[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[m][jt] = f32x16{};

    // the prologue's steps in order: the waits the compiler puts before
    // each step's first use of its weight registers count the loads issued
    // after them, and take the smallest count over the loop's entry and back
    // edge - a scale load scheduled behind the next steps' loads here would
    // shorten the prefetch of every iteration
    static_assert(kMmLead == 2, "the prologue issues kMmLead steps");
    t.template issue<0>(0);
    compiler_fence();
    t.template issue<1>(min(1, steps - 1));
    compiler_fence();

    auto body = [&](auto stage_c, int ks) {
      constexpr int S = decltype(stage_c)::value;
      stage_release_barrier();                               // every wave is done with step ks-1's stage
      // Always kMmLead steps ahead, so that every path has the same loads in
      // flight (the last ones re-read the final step into a free stage).
      t.template issue<(S + kMmLead) % kMmStages>(min(ks + kMmLead, steps - 1));
      wait_vm<kMmLead * LPS>();
      step_barrier();                                        // step ks's operand rows are in LDS
      const uint8_t* stage = S == 0 ? s_x0 : (S == 1 ? s_x1 : (S == 2 ? s_x2 : s_x3));
      bf16x8 af[NMAT][4];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) dequant_frags(t.wc[S][m], t.wsv[S][m], af[m]);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt < mtiles) {
          const int row = jt * 32 + l32;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int c = (half * 4 + kk) ^ ((row >> 1) & 7);
            const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(stage + row * (kMmK * 2) + c * 16);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
              acc[m][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m][kk], bfr, acc[m][jt], 0, 0, 0);
          }
        }
      }
    };
    // whole groups of four steps in the loop (one pattern of loads in flight
    // at the back edge, so the compiler's own waits stay as loose as ours),
    // then the remainder
    int s0 = 0;
    for (; s0 + kMmStages <= steps; s0 += kMmStages) {
      body(std::integral_constant<int, 0>{}, s0);
      body(std::integral_constant<int, 1>{}, s0 + 1);
      body(std::integral_constant<int, 2>{}, s0 + 2);
      body(std::integral_constant<int, 3>{}, s0 + 3);
    }
    if (s0 < steps) body(std::integral_constant<int, 0>{}, s0);
    if (s0 + 1 < steps) body(std::integral_constant<int, 1>{}, s0 + 1);
    if (s0 + 2 < steps) body(std::integral_constant<int, 2>{}, s0 + 2);
    wait_vm<0>();                                            // the surplus loads have landed
    __syncthreads();                                         // every wave is done with the operand stages

    // Epilogue, through LDS: per 32 x 32 block a lane holds 4 runs of 4
    // consecutive weight rows 8*q + 4*(lane/32) + 0..3 for one route column,
    // i.e. 8-byte pieces of 32 different output rows per store.  They are
    // written to LDS first, one stage per route tile jt (32 routes x the
    // workgroup's rows), the 16-byte chunk c of route r at position
    // c ^ (r % chunks), so that 16 consecutive routes hit 16 different bank
    // groups; then every wave stores whole contiguous runs of one route's
    // output row (16 bytes per lane).
    constexpr int kChunks = kWgRows / 8;                     // 16-byte chunks of one route's rows in the tile
    constexpr int kRouteBytes = kWgRows * 2;
    static_assert(32 * kRouteBytes <= kMmStageBytes, "a route tile's outputs fit one operand stage");
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < mtiles) {
        uint8_t* st = jt == 0 ? s_x0 : (jt == 1 ? s_x1 : (jt == 2 ? s_x2 : s_x3));
        uint8_t* rowp = st + l32 * kRouteBytes + half * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (GU) {
            const float Gg = sload(p.gsc, e * 3 + 0), Gu = sload(p.gsc, e * 3 + 1);
            uint32_t hv[2];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const float g0 = acc[0][jt][4 * q + 2 * t2] * Gg, g1 = acc[0][jt][4 * q + 2 * t2 + 1] * Gg;
              const float u0 = acc[1][jt][4 * q + 2 * t2] * Gu, u1 = acc[1][jt][4 * q + 2 * t2 + 1] * Gu;
              hv[t2] = f32_to_bf16_rne(silu(g0) * u0) | (f32_to_bf16_rne(silu(g1) * u1) << 16);
            }
            const int c = wave * 4 + q;
            *reinterpret_cast<uint2*>(rowp + ((c ^ (l32 % kChunks)) * 16)) = make_uint2(hv[0], hv[1]);
          } else {
            const float Gd = sload(p.gsc, e * 3 + 2);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              const int c = m * (kMmRows / 8) + wave * 4 + q;
              *reinterpret_cast<uint2*>(rowp + ((c ^ (l32 % kChunks)) * 16)) =
                  make_uint2(f32_to_f16_bits(acc[m][jt][4 * q] * Gd) | (f32_to_f16_bits(acc[m][jt][4 * q + 1] * Gd) << 16),
                             f32_to_f16_bits(acc[m][jt][4 * q + 2] * Gd) | (f32_to_f16_bits(acc[m][jt][4 * q + 3] * Gd) << 16));
            }
          }
        }
      }
    }
    __syncthreads();
    uint16_t* const out = GU ? p.h : p.o;
    const int total = mc * kChunks;
    for (int idx = tid; idx < total; idx += kMmThreads) {
      const int r = idx / kChunks, j = idx % kChunks;        // route of the chunk, its position in LDS
      const int c = j ^ (r % 32 % kChunks);                  // the output chunk stored there
      const int n = n0 + c * 8;
      if (n >= N) continue;                                  // N is a multiple of 32: whole chunks
      const int jt = r >> 5;
      const uint8_t* st = jt == 0 ? s_x0 : (jt == 1 ? s_x1 : (jt == 2 ? s_x2 : s_x3));
      const uint4 v = *reinterpret_cast<const uint4*>(st + (r & 31) * kRouteBytes + j * 16);
      *reinterpret_cast<uint4*>(out + (size_t)(off + m0 + r) * N + n) = v;
    }
  }
}

// Streaming form of the packed down tiles, for large batches (their items
// outnumber the CU slots several times): one workgroup per CU slot takes
// units - one row tile of one item - from a counter per XCD class until the
// list is done.  Workgroup b counts in class b % 8 (the XCD it is dealt to),
// and unit u of class c is row tile u % tiles_n of item (u / tiles_n) * 8 + c,
// so an item's tiles stay on one XCD and each class walks the list longest
// first, as the one-unit-per-workgroup grid does.  The next unit is claimed
// at the current unit's first step and set up at its fifth; its first
// kMmLead steps are issued during the current unit's last ones (the one-unit
// grid re-reads the final step there), so the next unit's head - the list
// entry, the first operand bytes - overlaps the current unit's last steps
// and epilogue, and no workgroup is dispatched per unit.  The epilogue runs
// one route tile at a time through stage 3, which holds no prefetched rows.
// K must run a multiple of four steps, at least eight.  The workgroup that
// finishes last clears the counters for the next launch.
constexpr int kQueueStride = kWlQueueStride;             // ints per counter (one 128-byte line each)
static_assert(kWlQueueInts == (kXcds + 1) * kQueueStride, "8 class counters, then the finished count");

// One lane's claim: an offset the compiler cannot see is zero keeps its
// atomic optimizer from turning the add into a wave-wide one whose result it
// reads at once (a wait for every load in flight).
__device__ __forceinline__ int atomic_claim(int32_t* c) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return __hip_atomic_fetch_add(c + z, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ties a ring entry to the program point: its conversion cannot be scheduled
// before this (after the step's wait, and so after the next step's loads).
__device__ __forceinline__ void pin(uint4& w, uint16_t& s) {
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w), "+v"(s));
}

template <int NSUB>
__global__ __launch_bounds__(kMmThreads, 2) void ffn_mfma_down_stream_kernel(FfnParams p, int32_t* queue) {
  using Tile = MmTile<false, true, NSUB>;
  constexpr int kWgRows = kMmRows * NSUB;
  constexpr int LPS = Tile::kLoadsPerStep;
  __shared__ __align__(16) uint8_t s_x0[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x1[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x2[kMmStageBytes];
  __shared__ __align__(16) uint8_t s_x3[kMmStageBytes];
  __shared__ int s_unit;                                     // the claimed unit
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int N = p.H, K = p.I;
  const int tiles_n = (N + kWgRows - 1) / kWgRows;
  const int steps = K / kMmK;
  const int cls = blockIdx.x % kXcds;
  int32_t* const ctr = queue + cls * kQueueStride;
  const int n_items = min(sload(p.plan_down, 0), p.plan_max);
  const int R = p.T * p.k;
  const size_t mat = packed_matrix_bytes(N, K), codes = packed_code_bytes(N, K);
  const uint8_t* const mbase = p.packed + 2 * (size_t)p.E * packed_matrix_bytes(p.I, p.H);

  // unit u of this class: expert, first bucket position, routes, first row;
  // cnt = 0 past the list
  struct Unit {
    int e, off, cnt, n0;
  };
  auto unit_of = [&](int u) {
    Unit w = {0, 0, 0, 0};
    const int it = (u / tiles_n) * kXcds + cls;
    if (u >= 0 && it < n_items) {
      w.e = min(max(sload(p.plan_down, 4 + 4 * it), 0), p.E - 1);
      w.off = min(max(sload(p.plan_down, 5 + 4 * it), 0), R);
      w.cnt = min(max(sload(p.plan_down, 6 + 4 * it), 0), min(kMmRoutes, R - w.off));
      w.n0 = (u % tiles_n) * kWgRows;
    }
    return w;
  };
  Tile t;
  t.s_x[0] = s_x0;
  t.s_x[1] = s_x1;
  t.s_x[2] = s_x2;
  t.s_x[3] = s_x3;
  t.wave = wave;
  t.lane = lane;
  // the unit's weight tiles and h rows (rows past its routes repeat its last)
  auto point_at = [&](const Unit& w) {
#pragma unroll
    for (int m = 0; m < NSUB; ++m) {
      const uint8_t* me = mbase + (size_t)w.e * mat;
      t.rc[m] = make_rsrc(me, (uint32_t)codes);
      t.rs[m] = make_rsrc(me + codes, (uint32_t)(mat - codes));
      const uint32_t tile_step0 = (uint32_t)(w.n0 / kMmRows + m) * (uint32_t)steps;
      t.w_voff[m] = (uint32_t)(wave * 64 + lane) * 16 + tile_step0 * 4096u;
      t.s_voff[m] = (uint32_t)(wave * 64 + lane) * 2 + tile_step0 * 512u;
    }
    t.rb = make_rsrc(p.h + (size_t)w.off * p.I, (uint32_t)w.cnt * (uint32_t)p.I * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = (i * 4 + wave) * 64 + lane;
      const int row = q >> 3, c = (q & 7) ^ ((row >> 1) & 7);
      t.x_goff[i] = (uint32_t)min(row, w.cnt - 1) * (uint32_t)K * 2u + (uint32_t)c * 16;
    }
  };

  if (tid == 0) s_unit = atomic_claim(ctr);
  __syncthreads();
  Unit cur = unit_of(__builtin_amdgcn_readfirstlane(s_unit));
  if (cur.cnt > 0) {
    point_at(cur);
    static_assert(kMmLead == 2, "the prologue issues kMmLead steps");
    t.template issue<0>(0);
    compiler_fence();
    t.template issue<1>(1);
    compiler_fence();
    for (;;) {
      const int mtiles = (cur.cnt + 31) >> 5;
      Unit nxt = {0, 0, 0, 0};
      int claimed = 0;
      f32x16 acc[NSUB][4];
#pragma unroll
      for (int m = 0; m < NSUB; ++m)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[m][jt] = f32x16{};

      auto body = [&](auto stage_c, int ks) {
        constexpr int S = decltype(stage_c)::value;
        stage_release_barrier();                             // every wave is done with step ks-1's stage
        if (ks == 4) nxt = unit_of(__builtin_amdgcn_readfirstlane(s_unit));   // claimed at step 0
        if (ks == steps - kMmLead && nxt.cnt > 0) point_at(nxt);
        // kMmLead steps ahead: the current unit's, then the next unit's
        // first ones, or (no next unit) the final step again into a free stage
        const int is = ks + kMmLead < steps ? ks + kMmLead : (nxt.cnt > 0 ? ks + kMmLead - steps : steps - 1);
        t.template issue<(S + kMmLead) % kMmStages>(is);
        if (ks == 0 && tid == 0) claimed = atomic_claim(ctr);
        wait_vm<kMmLead * LPS>();
        step_barrier();                                      // step ks's operand rows are in LDS
        if (ks == 3 && tid == 0) s_unit = claimed;
        const uint8_t* stage = S == 0 ? s_x0 : (S == 1 ? s_x1 : (S == 2 ? s_x2 : s_x3));
        bf16x8 af[NSUB][4];
#pragma unroll
        for (int m = 0; m < NSUB; ++m) {
          pin(t.wc[S][m], t.wsv[S][m]);
          dequant_frags(t.wc[S][m], t.wsv[S][m], af[m]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          if (jt < mtiles) {
            const int row = jt * 32 + l32;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const int c = (half * 4 + kk) ^ ((row >> 1) & 7);
              const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(stage + row * (kMmK * 2) + c * 16);
#pragma unroll
              for (int m = 0; m < NSUB; ++m)
                acc[m][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m][kk], bfr, acc[m][jt], 0, 0, 0);
            }
          }
        }
      };
      for (int s0 = 0; s0 < steps; s0 += kMmStages) {
        body(std::integral_constant<int, 0>{}, s0);
        body(std::integral_constant<int, 1>{}, s0 + 1);
        body(std::integral_constant<int, 2>{}, s0 + 2);
        body(std::integral_constant<int, 3>{}, s0 + 3);
      }

      // Epilogue through stage 3 (the final step's, the only one without
      // prefetched rows), one route tile per pass: o = fp16(Gd * acc) to LDS
      // as in the one-unit kernel, then every wave stores whole runs of one
      // route's output row.
      constexpr int kChunks = kWgRows / 8;
      constexpr int kRouteBytes = kWgRows * 2;
      static_assert(32 * kRouteBytes <= kMmStageBytes, "a route tile's outputs fit one operand stage");
      const float Gd = sload(p.gsc, cur.e * 3 + 2);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt < mtiles) {
          stage_release_barrier();                           // stage 3 is free (step reads or the previous pass)
          uint8_t* rowp = s_x3 + l32 * kRouteBytes + half * 8;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int m = 0; m < NSUB; ++m) {
              const int c = m * (kMmRows / 8) + wave * 4 + q;
              *reinterpret_cast<uint2*>(rowp + ((c ^ (l32 % kChunks)) * 16)) =
                  make_uint2(f32_to_f16_bits(acc[m][jt][4 * q] * Gd) | (f32_to_f16_bits(acc[m][jt][4 * q + 1] * Gd) << 16),
                             f32_to_f16_bits(acc[m][jt][4 * q + 2] * Gd) | (f32_to_f16_bits(acc[m][jt][4 * q + 3] * Gd) << 16));
            }
          }
          // the tile's outputs are in LDS: each wave's writes have landed
          // before the barrier (it does not wait for them by itself)
          stage_release_barrier();
          const int rc = min(32, cur.cnt - jt * 32);
          for (int idx = tid; idx < rc * kChunks; idx += kMmThreads) {
            const int r = idx / kChunks, j = idx % kChunks;
            const int c = j ^ (r % kChunks);
            const int n = cur.n0 + c * 8;
            if (n >= N) continue;                            // N is a multiple of 32: whole chunks
            const uint4 v = *reinterpret_cast<const uint4*>(s_x3 + r * kRouteBytes + j * 16);
            *reinterpret_cast<uint4*>(p.o + (size_t)(cur.off + jt * 32 + r) * N + n) = v;
          }
        }
      }
      if (nxt.cnt <= 0) break;
      cur = nxt;
    }
    wait_vm<0>();                                            // the final re-reads have landed in LDS
  }
  // the last workgroup to finish clears the counters
  if (tid == 0 && atomic_claim(queue + kXcds * kQueueStride) == (int)gridDim.x - 1) {
    for (int c = 0; c <= kXcds; ++c)
      __hip_atomic_store(queue + c * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ work lists

static_assert(kMmRoutes == kWlRoutes, "an MFMA item is one route chunk of the MFMA kernels");

// The work lists (work_list.h) from the bucket arrays, one expert slot per
// thread (S <= 1024 slots); the active list holds -1 past its end, so
// n_active is not needed.  moe_step builds the same lists in its bucketing
// kernel and skips this one.
__global__ __launch_bounds__(kWlThreads) void plan_kernel(FfnParams p) {
  __shared__ WorkListShared sh;
  const int tid = threadIdx.x;
  const int S = min(p.E, p.T * p.k);
  int e = -1, off = 0, cnt = 0;
  if (tid < S) {
    e = slot_expert(p, tid);
    if (e >= 0) expert_routes(p, e, off, cnt);
  }
  WorkLists wl;
  wl.plan = p.plan;
  wl.rd_list = p.rd_list;
  wl.plan_max = p.plan_max;
  wl.mfma_min = p.mfma_min;
  wl.rd_plan = p.rd_plan;
  wl.queues = p.queues;
  wl.split_items = p.split_items;
  wl.plan_down = p.plan_down;
  build_work_lists(wl, sh, e, cnt, off);
}

// ------------------------------------------------------------------ combine

constexpr int kCombineCols = 8 * kThreads;   // output columns per workgroup
constexpr int kMaxK = 32;

// y[t, c..c+7] = sum over slots j in order of w[t,j] * o[route_pos[t*k+j], c..c+7],
// in fp32 from the routes' fp16 down outputs (each route's result is rounded
// once to fp16 before the fp32 weighting, as the SM70 design note's
// contract keeps it: page "Persistent execution for Flash-Next GGUF on
// SM70", section "First implementation boundary", step 4).  One workgroup
// per (token, 2048 columns): the token's weights and route positions are
// staged once, then every o load (16 bytes per thread) is issued before the
// sum.
__global__ __launch_bounds__(kThreads) void combine_kernel(FfnParams p) {
  __shared__ float s_w[kMaxK];
  __shared__ int s_pos[kMaxK];
  const int col_blocks = (p.H + kCombineCols - 1) / kCombineCols;
  const int t = blockIdx.x / col_blocks;
  const int c = (blockIdx.x - t * col_blocks) * kCombineCols + 8 * threadIdx.x;
  const int R = p.T * p.k;
  if (threadIdx.x < p.k) {
    s_w[threadIdx.x] = p.topk_w[(size_t)t * p.k + threadIdx.x];
    s_pos[threadIdx.x] = min(max(p.route_pos[(size_t)t * p.k + threadIdx.x], 0), R - 1);
  }
  __syncthreads();
  if (c >= p.H) return;                        // H is a multiple of 32: c + 8 <= H
  uint4 ov[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < p.k) ov[j] = *reinterpret_cast<const uint4*>(p.o + (size_t)s_pos[j] * p.H + c);
  float yv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < p.k) {
      const uint32_t d[4] = {ov[j].x, ov[j].y, ov[j].z, ov[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yv[2 * q] = fmaf(s_w[j], f16_bits_to_f32(d[q] & 0xFFFFu), yv[2 * q]);
        yv[2 * q + 1] = fmaf(s_w[j], f16_bits_to_f32(d[q] >> 16), yv[2 * q + 1]);
      }
    }
  }
  uint32_t yb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) yb[q] = f32_to_bf16_rne(yv[2 * q]) | (f32_to_bf16_rne(yv[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(p.y + (size_t)t * p.H + c) = make_uint4(yb[0], yb[1], yb[2], yb[3]);
}

// ------------------------------------------------------------------ down + combine (small batches)

constexpr int kDcMaxRoutes = 128;          // T*k on the fused down/combine path
constexpr int kDcMaxLds = 65536;           // all routes' h and o staged in LDS up to this size
constexpr int kDcThreads = 1024;           // sixteen waves share one row block
constexpr int kDcWaves = kDcThreads / kWave;
constexpr int kDcLoadsPerSlot = 2;         // one b128 code load and one b16 scale load
constexpr int kDcHLoads = kDcMaxLds / 16 / kDcThreads;   // 16-byte h pieces per thread
// Shared-expert down row `row` (weights w: NC chunks of this lane) for every
// token, its h read from LDS (s_hs: [T, Is] bf16): the products and the
// fixed-order lane sum of se_down_rows, kSeTokens tokens' sums in flight
// together.
template <int NC>
__device__ __forceinline__ void se_down_row_lds(const SharedRows& sr, const u32x4 (&wv)[2], const uint8_t* s_hs,
                                                int row, int lane) {
  // the row's registers pass through an empty asm statement before the token
  // loop, so that the wait for its loads is placed here, in straight-line
  // code, with an exact count (for a use inside the loop the compiler waits
  // for every load in flight, the slots' weight rows included)
  u32x4 w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    w[c] = wv[c];
    asm volatile("" : "+v"(w[c]));
  }
  const size_t rb = (size_t)sr.Is * 2;
  auto pass = [&](int t0) {
    float acc[kSeTokens];
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) {
      const uint8_t* hr = s_hs + (size_t)min(t0 + j, sr.T - 1) * rb + (size_t)lane * 16;
      u32x4 hv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) hv[c] = *reinterpret_cast<const u32x4*>(hr + c * 64 * 16);
      acc[j] = se_dot<NC>(w, hv);
    }
#pragma unroll
    for (int j = 0; j < kSeTokens; ++j) {
      const float ys = wave_sum_xor(acc[j]);
      if (lane == 0 && t0 + j < sr.T && row < sr.H) sr.y[(size_t)(t0 + j) * sr.H + row] = (uint16_t)f32_to_bf16_rne(ys);
    }
  };
  // up to kSeTokens tokens (the decode batches) in straight-line code: in a
  // loop the compiler would wait for every load in flight before its first
  // iteration, the slots' weight rows included
  if (sr.T <= kSeTokens) {
    pass(0);
  } else {
    for (int t0 = 0; t0 < sr.T; t0 += kSeTokens) pass(t0);
  }
}

// Byte offset of a shared expert's h in the route-slot down/unroute's LDS:
// after the routes' h ([R, I] bf16) and o ([R, rpw] fp32), 16-byte aligned.
__host__ __device__ inline size_t dc_se_h_offset(int R, int I, int rpw) {
  return ((size_t)R * I * 2 + (size_t)R * rpw * 4 + 15) & ~(size_t)15;
}

// Down projection and weighted unroute of a small batch in one kernel, with
// the work split by output rows instead of by expert: workgroup b owns rows
// [b*rpw, b*rpw + rpw) of y (rpw = 64 / lanes per row) for every token.  Its
// sixteen waves take the active slots a = wave + 16*u, u < SLOTS (SLOTS =
// ceil(slots / 16), so one pass covers them all), and hold one 16-byte chunk
// per lane of each slot's rows of W_down: many waves with few loads each keep
// more row pieces in flight than few waves with many.  o[route, row] stays in
// LDS, and each token's routes are finally summed in slot order.  No o round
// trip through memory and no cross-workgroup ordering.
//
// Issue order: all routes' h rows (up to kDcHLoads 16-byte pieces per thread
// into registers), the routes' positions and weights, the slots' expert ids
// (scalar path), then every slot's weight row, and then route ranges and
// global scales through the scalar path.  Every vector load is issued
// unconditionally - a piece or slot past the end reads out of range, which
// returns zeros without memory traffic - so the loads land in a fixed order.
// h goes to LDS as soon as it has landed, the waves meet at a barrier that
// does not drain the weight loads, and each wave computes slot by slot as
// their rows arrive (vector loads complete in order).  All of them are
// ordinary buffer loads and none sits in a loop, which keeps the compiler's
// wait counts exact (with LDS-direct loads in flight as well it waits for
// everything).
//
// Route slots (RS, after select_gate_up_kernel): slot a is route a itself
// (expert topk_idx[a], h row a, one route), so the buckets are not needed.
// A shared expert's down rows can ride along there (SE): the last rpw waves
// each take output row row0 + i of it, loading that weight row ahead of
// their slots' rows and summing it first; the shared h (T x Is bf16) is
// staged in LDS behind o with the routes' h.  Each row is summed as
// se_down_rows sums it.
template <int LD, int SLOTS, bool RS = false, bool SE = false>
__global__ __launch_bounds__(kDcThreads, SLOTS <= 4 ? 2 : 1) void down_combine_kernel(FfnParams p) {
  static_assert(RS || !SE, "shared rows ride along in route-slot mode only");
  extern __shared__ __align__(16) uint8_t s_dyn8[];   // [R, I] bf16 h, then [R, rpw] fp32 o
  __shared__ int s_src[kDcMaxRoutes];
  __shared__ float s_w[kDcMaxRoutes];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = p.T * p.k;
  const int ld = LD ? LD : p.lr_d, rpw = kWave / ld, sub = lane / ld, sl = lane & (ld - 1);
  const int row0 = blockIdx.x * rpw;
  const int S = RS ? R : min(p.E, R);
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn8);
  float* s_o = reinterpret_cast<float*>(s_dyn8 + (size_t)R * p.I * 2);

  // h rows of every route: piece q = tid + i*kDcThreads of the [R, I] block
  const uint32_t h_bytes = (uint32_t)R * p.I * 2;
  const auto rh = make_rsrc(p.h, h_bytes);
  u32x4 hv[kDcHLoads];
#pragma unroll
  for (int i = 0; i < kDcHLoads; ++i) {
    // a wave whose pieces all lie past h issues no load (address work is
    // not free); a partly covered wave reads zeros past the end
    hv[i] = u32x4{0u, 0u, 0u, 0u};
    if ((uint32_t)(wave * kWave + i * kDcThreads) * 16 < h_bytes)
      hv[i] = __builtin_amdgcn_raw_buffer_load_b128(rh, (uint32_t)(tid + i * kDcThreads) * 16, 0, 0);
  }
  // the shared expert's h, one piece per thread, and the shared down row of
  // each of the last rpw waves (one or two chunks per lane), ahead of the
  // routes' weights
  const uint32_t se_hbytes = SE ? (uint32_t)p.T * (uint32_t)p.sr.Is * 2u : 0u;
  const int se_w0 = kDcWaves - rpw;
  const bool se_wave = SE && wave >= se_w0;
  const int se_row = row0 + wave - se_w0;
  u32x4 se_hv = u32x4{0u, 0u, 0u, 0u};
  u32x4 se_w[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  if constexpr (SE) {
    // issued by every thread, past the buffer where there is nothing to read
    // (zeros, no memory traffic), so that the wait counts stay exact
    constexpr uint32_t kOff = 0x80000000u;
    se_hv = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(p.sr.h, se_hbytes),
                                                  (uint32_t)tid * 16 < se_hbytes ? (uint32_t)tid * 16 : kOff, 0, 0);
    const uint32_t se_rb = (uint32_t)p.sr.Is * 2u;
    const auto rsd = make_rsrc(p.sr.wd, (uint32_t)p.H * se_rb);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      se_w[c] = __builtin_amdgcn_raw_buffer_load_b128(
          rsd, se_wave && c < p.sr.dn_nc ? (uint32_t)se_row * se_rb + (uint32_t)(lane + 64 * c) * 16u : kOff, 0,
          kStreamAux);
  }
  // route positions and gate weights (an index past R re-reads the last)
  const int rt = min(tid, R - 1);
  const int src_r = RS ? rt : p.route_src[rt];
  const float w_r = p.topk_w[rt];
  compiler_fence();

  int e_u[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int a = wave + u * kDcWaves;
    if constexpr (RS) e_u[u] = a < S ? min(max(sload(p.topk_idx, a), 0), p.E - 1) : -1;
    else e_u[u] = a < S ? slot_expert(p, a) : -1;
  }
  const uint32_t code_row = (uint32_t)p.I / 2, scale_row = (uint32_t)p.I / 16;
  // one resource spans all of W_down (and one its scales); the host checks
  // that their byte counts fit 31 bits
  const auto rd = make_rsrc(p.wd, (uint32_t)p.E * p.H * code_row);
  const auto rds = make_rsrc(p.sd, (uint32_t)p.E * p.H * scale_row);
  const uint32_t lane_c = (uint32_t)sub * code_row + (uint32_t)sl * 16;
  const uint32_t lane_s = (uint32_t)sub * scale_row + (uint32_t)sl * 2;
  constexpr uint32_t kOutOfRange = 0x80000000u;       // past both resources: reads zero
  uint4 cd[SLOTS];
  uint32_t vd[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const uint32_t r = (uint32_t)max(e_u[u], 0) * (uint32_t)p.H + (uint32_t)row0;
    const uint32_t oc = e_u[u] >= 0 ? lane_c + r * code_row : kOutOfRange;
    const uint32_t os = e_u[u] >= 0 ? lane_s + r * scale_row : kOutOfRange;
    cd[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rd, oc, 0, kStreamAux));
    vd[u] = __builtin_amdgcn_raw_buffer_load_b16(rds, os, 0, kStreamAux);
  }
  compiler_fence();
  int off_u[SLOTS], cnt_u[SLOTS];
  float gd_u[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    off_u[u] = 0;
    cnt_u[u] = 0;
    gd_u[u] = 0.0f;
    if (e_u[u] >= 0) {
      if constexpr (RS) {
        off_u[u] = wave + u * kDcWaves;     // the route itself: h row a, one route
        cnt_u[u] = 1;
      } else {
        expert_routes(p, e_u[u], off_u[u], cnt_u[u]);
      }
      gd_u[u] = sload(p.gsc, e_u[u] * 3 + 2);
    }
  }
  // h and the route data were issued before the weight loads
#pragma unroll
  for (int i = 0; i < kDcHLoads; ++i) {
    const uint32_t q = (uint32_t)(tid + i * kDcThreads) * 16;
    if (q < h_bytes) *reinterpret_cast<u32x4*>(s_dyn8 + q) = hv[i];
  }
  if (tid < R) {
    s_src[tid] = min(max(src_r, 0), R - 1);
    s_w[tid] = w_r;
  }
  uint8_t* const s_hs = s_dyn8 + dc_se_h_offset(R, p.I, rpw);   // the shared expert's h
  if (SE && (uint32_t)tid * 16 < se_hbytes) *reinterpret_cast<u32x4*>(s_hs + tid * 16) = se_hv;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();                // h of every route is in LDS; weights still in flight
  compiler_fence();

  if (se_wave) {
    // y_shared[t, se_row] = bf16(W_down[se_row] . h_shared[t]), as se_down_rows
    // sums it; its row was loaded ahead of the slots' rows
    if (p.sr.dn_nc == 1) se_down_row_lds<1>(p.sr, se_w, s_hs, se_row, lane);
    else se_down_row_lds<2>(p.sr, se_w, s_hs, se_row, lane);
  }

  const bool row_ok = row0 + sub < p.H;
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    if (e_u[u] < 0) continue;
    for (int t = 0; t < cnt_u[u]; ++t) {
      const int pos = off_u[u] + t;
      const float one = opaque_one();
      uint32_t hr[16];
      load_operand_chunk(s_h + (size_t)pos * p.I, sl, hr);
      const float acc = dot_chunk(cd[u], vd[u], hr, 0.0f, one);
      const float v = (LD == 16 ? row16_sum(acc) : group_sum(acc, ld)) * gd_u[u];
      if (sl == 0 && row_ok) s_o[s_src[pos] * rpw + sub] = v;
    }
  }
  __syncthreads();

  // y[t, row0 + r] = sum over slots j in order of w[t,j] * o[route_pos[t,j], r]
  for (int i = tid; i < p.T * rpw; i += kDcThreads) {
    const int t = i / rpw, r = i - t * rpw;
    if (row0 + r >= p.H) continue;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j) acc = fmaf(s_w[t * p.k + j], s_o[(t * p.k + j) * rpw + r], acc);
    p.y[(size_t)t * p.H + row0 + r] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

template <int LD, bool RS = false, bool SE = false>
void launch_down_combine(const FfnParams& p, unsigned grid, size_t dyn, int slots, hipStream_t s) {
  const int per_wave = (slots + kDcWaves - 1) / kDcWaves;
  if (per_wave <= 1) down_combine_kernel<LD, 1, RS, SE><<<grid, kDcThreads, dyn, s>>>(p);
  else if (per_wave == 2) down_combine_kernel<LD, 2, RS, SE><<<grid, kDcThreads, dyn, s>>>(p);
  else if (per_wave == 3) down_combine_kernel<LD, 3, RS, SE><<<grid, kDcThreads, dyn, s>>>(p);
  else if (per_wave == 4) down_combine_kernel<LD, 4, RS, SE><<<grid, kDcThreads, dyn, s>>>(p);
  else down_combine_kernel<LD, kDcMaxRoutes / kDcWaves, RS, SE><<<grid, kDcThreads, dyn, s>>>(p);
}

// ------------------------------------------------------------------ rows of several chunks per lane

// Row-dot kernels for row lengths whose 16-byte chunk count C = cols/32 is
// not a power of two up to 64 (H = 2560 and I = 640 of the Flash-Next expert
// give C = 80 and 20; H = 4096 gives 128).  kNcLanes lanes share a row and
// lane sl reads chunks sl, sl + 16, ..., sl + 16*(NC-1), NC = ceil(C / 16);
// a chunk index past the row (the tail) is given an offset past the buffer
// resource, which reads zero codes and zero scales, so it adds exactly zero
// to the dot product (its operand chunk is read clamped to the last chunk of
// the row: finite, and never past the buffer).  Scales are read per chunk
// (two bytes) next to its codes; each unit's products follow the same
// dot_chunk and fixed-order lane sums as the one-chunk kernels.
constexpr int kNcLanes = 16;                 // lanes per row
constexpr int kNcRowsPerWave = kWave / kNcLanes;
constexpr uint32_t kNcOutOfRange = 0x80000000u;

// Offsets of chunk i of this lane in a row of C chunks starting at byte
// `row_code` (codes) / `row_scale` (scales); kNcOutOfRange past the row.
__device__ __forceinline__ void nc_chunk_offsets(int sl, int i, int C, uint32_t row_code, uint32_t row_scale,
                                                 bool row_ok, uint32_t& oc, uint32_t& os) {
  const int c = sl + i * kNcLanes;
  const bool ok = row_ok && c < C;
  oc = ok ? row_code + (uint32_t)c * 16u : kNcOutOfRange;
  os = ok ? row_scale + (uint32_t)c * 2u : kNcOutOfRange;
}

// Gate and up rows of one tile (kWavesPerBlock * kNcRowsPerWave = 16 rows of
// I) for all routes of expert e, one row per 16-lane group.
template <int NC>
__global__ __launch_bounds__(kThreads, 2) void gate_up_nc_kernel(FfnParams p, int n_tasks) {
  constexpr int kRpt = kWavesPerBlock * kNcRowsPerWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / kNcLanes, sl = lane & (kNcLanes - 1);
  const int tiles = (p.I + kRpt - 1) / kRpt;
  const int task = blockIdx.x;
  if (task >= n_tasks) return;
  const int a = task / tiles, tile = task - a * tiles;
  const int e = row_dot_expert(p, a);
  if (e < 0) return;
  const int C = p.H / 32;
  const uint32_t code_row = (uint32_t)p.H / 2, scale_row = (uint32_t)p.H / 16;
  const uint32_t mat_codes = (uint32_t)p.I * code_row, mat_scales = (uint32_t)p.I * scale_row;
  const auto rg = make_rsrc(p.wg + (size_t)e * mat_codes, mat_codes);
  const auto ru = make_rsrc(p.wu + (size_t)e * mat_codes, mat_codes);
  const auto rsg = make_rsrc(p.sg + (size_t)e * mat_scales, mat_scales);
  const auto rsu = make_rsrc(p.su + (size_t)e * mat_scales, mat_scales);
  const int row = tile * kRpt + wave * kNcRowsPerWave + sub;
  const bool row_ok = row < p.I;
  uint4 cg[NC], cu[NC];
  uint32_t vg[NC], vu[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t oc, os;
    nc_chunk_offsets(sl, i, C, (uint32_t)row * code_row, (uint32_t)row * scale_row, row_ok, oc, os);
    cg[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rg, oc, 0, kStreamAux));
    cu[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(ru, oc, 0, kStreamAux));
    vg[i] = __builtin_amdgcn_raw_buffer_load_b16(rsg, os, 0, kStreamAux);
    vu[i] = __builtin_amdgcn_raw_buffer_load_b16(rsu, os, 0, kStreamAux);
  }
  compiler_fence();
  int off, cnt;
  expert_routes(p, e, off, cnt);
  const float Gg = sload(p.gsc, e * 3 + 0), Gu = sload(p.gsc, e * 3 + 1);
  for (int r = 0; r < cnt; ++r) {
    const int pos = off + r;
    const int tok = min(max(sload(p.route_src, pos) / p.k, 0), p.T - 1);
    const uint16_t* xrow = p.x + (size_t)tok * p.H;
    const float one = opaque_one();
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      uint32_t xr[16];
      load_operand_chunk(xrow, min(sl + i * kNcLanes, C - 1), xr);
      ag = dot_chunk(cg[i], vg[i], xr, ag, one);
      au = dot_chunk(cu[i], vu[i], xr, au, one);
    }
    const float gs = row16_sum(ag) * Gg, us = row16_sum(au) * Gu;
    if (sl == 0 && row_ok) p.h[(size_t)pos * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
  }
}

// The small step for gate/up rows of several chunks per lane (H = 2560: 80
// chunks, the Flash-Next expert): as select_gate_up_kernel - workgroup
// (route r, 16 rows of I), r = t*k + j, selects token t's j-th expert itself
// (wave 0 runs the selection rounds up to round j) and computes that tile
// for that one route, h[r, rows] by flat route id; the launch's last
// workgroup writes every routing output - with gate_up_nc_kernel's rows
// (kNcLanes lanes per row, NC chunks per lane).  Token t's activation row
// goes to LDS while wave 0 selects: it does not depend on the routing.
constexpr int kSgNcXBytes = 8192;            // one activation row, H <= 4096

template <int V, int KC, int NC>
__global__ __launch_bounds__(kThreads, 2) void select_gate_up_nc_kernel(FfnParams p, const float* __restrict__ logits,
                                                                        const float* __restrict__ bias,
                                                                        int32_t* __restrict__ topk_idx,
                                                                        float* __restrict__ topk_w, int n_tasks) {
  constexpr int kRpt = kWavesPerBlock * kNcRowsPerWave;
  constexpr int kXLoads = kSgNcXBytes / 16 / kThreads;
  __shared__ __align__(16) uint8_t s_x[kSgNcXBytes];
  __shared__ int s_e;
  const int task = blockIdx.x;
  if (task >= n_tasks) {
    // the launch's last workgroup: every routing output
    small_route_bucket<V, KC>(p, logits, bias, topk_idx, topk_w);
    return;
  }
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane / kNcLanes, sl = lane & (kNcLanes - 1);
  const int tiles = (p.I + kRpt - 1) / kRpt;
  const int r = task / tiles, tile = task - r * tiles;
  const int t = r / p.k, j = r - t * p.k;
  const int C = p.H / 32;
  // the activation row, 16 bytes per thread and pass (pieces past the row
  // read zeros and are not stored)
  const uint32_t x_bytes = (uint32_t)p.H * 2;
  const auto rx = make_rsrc(p.x + (size_t)t * p.H, x_bytes);
  u32x4 xv[kXLoads];
#pragma unroll
  for (int q = 0; q < kXLoads; ++q)
    xv[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + q * kThreads) * 16, 0, 0);
  compiler_fence();
  if (wave == (int)(blockIdx.x & (kWavesPerBlock - 1))) {
    // only slot j's expert: the rounds of the selection up to round j (the
    // selecting wave rotates with the workgroup, as in select_gate_up_kernel)
    const int e_j = select_slot<V, KC>(logits + (size_t)t * p.E, bias, p.E, j, lane);
    if (lane == 0) s_e = e_j;
  }
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    const uint32_t o = (uint32_t)(tid + q * kThreads) * 16;
    if (o < x_bytes) *reinterpret_cast<u32x4*>(s_x + o) = xv[q];
  }
  __syncthreads();
  const int e = min(max(__builtin_amdgcn_readfirstlane(s_e), 0), p.E - 1);

  // the tile's rows of expert e, as gate_up_nc_kernel
  const uint32_t code_row = (uint32_t)p.H / 2, scale_row = (uint32_t)p.H / 16;
  const uint32_t mat_codes = (uint32_t)p.I * code_row, mat_scales = (uint32_t)p.I * scale_row;
  const auto rg = make_rsrc(p.wg + (size_t)e * mat_codes, mat_codes);
  const auto ru = make_rsrc(p.wu + (size_t)e * mat_codes, mat_codes);
  const auto rsg = make_rsrc(p.sg + (size_t)e * mat_scales, mat_scales);
  const auto rsu = make_rsrc(p.su + (size_t)e * mat_scales, mat_scales);
  const int row = tile * kRpt + wave * kNcRowsPerWave + sub;
  const bool row_ok = row < p.I;
  uint4 cg[NC], cu[NC];
  uint32_t vg[NC], vu[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t oc, os;
    nc_chunk_offsets(sl, i, C, (uint32_t)row * code_row, (uint32_t)row * scale_row, row_ok, oc, os);
    cg[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rg, oc, 0, kStreamAux));
    cu[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(ru, oc, 0, kStreamAux));
    vg[i] = __builtin_amdgcn_raw_buffer_load_b16(rsg, os, 0, kStreamAux);
    vu[i] = __builtin_amdgcn_raw_buffer_load_b16(rsu, os, 0, kStreamAux);
  }
  compiler_fence();
  const float Gg = sload(p.gsc, e * 3 + 0), Gu = sload(p.gsc, e * 3 + 1);
  const float one = opaque_one();
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t xr[16];
    load_operand_chunk(reinterpret_cast<const uint16_t*>(s_x), min(sl + i * kNcLanes, C - 1), xr);
    ag = dot_chunk(cg[i], vg[i], xr, ag, one);
    au = dot_chunk(cu[i], vu[i], xr, au, one);
  }
  const float gs = row16_sum(ag) * Gg, us = row16_sum(au) * Gu;
  if (sl == 0 && row_ok) p.h[(size_t)r * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
}

// Down rows of one tile (16 rows of H) for all routes of expert e -> o (fp32).
template <int NC>
__global__ __launch_bounds__(kThreads, 2) void down_nc_kernel(FfnParams p, int n_tasks) {
  constexpr int kRpt = kWavesPerBlock * kNcRowsPerWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / kNcLanes, sl = lane & (kNcLanes - 1);
  const int tiles = (p.H + kRpt - 1) / kRpt;
  const int task = blockIdx.x;
  if (task >= n_tasks) return;
  const int a = task / tiles, tile = task - a * tiles;
  const int e = row_dot_expert(p, a);
  if (e < 0) return;
  const int C = p.I / 32;
  const uint32_t code_row = (uint32_t)p.I / 2, scale_row = (uint32_t)p.I / 16;
  const uint32_t mat_codes = (uint32_t)p.H * code_row, mat_scales = (uint32_t)p.H * scale_row;
  const auto rd = make_rsrc(p.wd + (size_t)e * mat_codes, mat_codes);
  const auto rds = make_rsrc(p.sd + (size_t)e * mat_scales, mat_scales);
  const int row = tile * kRpt + wave * kNcRowsPerWave + sub;
  const bool row_ok = row < p.H;
  uint4 cd[NC];
  uint32_t vd[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t oc, os;
    nc_chunk_offsets(sl, i, C, (uint32_t)row * code_row, (uint32_t)row * scale_row, row_ok, oc, os);
    cd[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rd, oc, 0, kStreamAux));
    vd[i] = __builtin_amdgcn_raw_buffer_load_b16(rds, os, 0, kStreamAux);
  }
  compiler_fence();
  int off, cnt;
  expert_routes(p, e, off, cnt);
  const float Gd = sload(p.gsc, e * 3 + 2);
  for (int r = 0; r < cnt; ++r) {
    const int pos = off + r;
    const uint16_t* hrow = p.h + (size_t)pos * p.I;
    const float one = opaque_one();
    float ad = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      uint32_t hr[16];
      load_operand_chunk(hrow, min(sl + i * kNcLanes, C - 1), hr);
      ad = dot_chunk(cd[i], vd[i], hr, ad, one);
    }
    const float v = row16_sum(ad) * Gd;
    if (sl == 0 && row_ok) p.o[(size_t)pos * p.H + row] = f32_to_f16_bits(v);
  }
}

// Down projection and weighted unroute of a small batch (the design of
// down_combine_kernel, rows of NC chunks per lane): workgroup b owns rows
// [4b, 4b + 4) of y for every token; its sixteen waves take the active slots
// a = wave + 16u, u < SLOTS; all routes' h and the o of its rows stay in LDS;
// each token's routes are summed in slot order.
// Eight waves per workgroup and exactly ceil(slots / 8) slots per wave (at
// most kDcNcMaxChunks chunks of weights per lane in flight): under 80
// registers three workgroups fit a CU, so a batch's row blocks (H / 4 of
// them) run in one round on 256 compute units up to H = 3072.
constexpr int kDcNcThreads = 512;
constexpr int kDcNcWaves = kDcNcThreads / kWave;
constexpr int kDcNcMaxChunks = 10;          // NC * SLOTS
constexpr int kDcNcHLoads = kDcMaxLds / 16 / kDcNcThreads;   // h pieces per thread at most

// LDS bytes of the h rows in down_combine_nc_kernel: whole kilobytes (one
// wave's piece of the buffer_load ... lds staging).
constexpr uint32_t dc_nc_h_lds(uint32_t h_bytes) { return (h_bytes + 1023u) & ~1023u; }

// Route slots (RS, after select_gate_up_nc_kernel): slot a is route a itself
// (expert topk_idx[a], h row a, one route), as in down_combine_kernel.
template <int NC, int SLOTS, bool RS = false>
__global__ __launch_bounds__(kDcNcThreads, 3) void down_combine_nc_kernel(FfnParams p) {
  extern __shared__ __align__(16) uint8_t s_dyn8[];   // [R, I] bf16 h (to a whole KB), then [R, 4] fp32 o
  __shared__ int s_src[kDcMaxRoutes];
  __shared__ float s_w[kDcMaxRoutes];
  constexpr int rpw = kNcRowsPerWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane / kNcLanes, sl = lane & (kNcLanes - 1);
  const int row0 = blockIdx.x * rpw;
  const int R = p.T * p.k;
  const int S = RS ? R : min(p.E, R);
  const int C = p.I / 32;
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn8);
  const uint32_t h_bytes = (uint32_t)R * p.I * 2;
  float* s_o = reinterpret_cast<float*>(s_dyn8 + dc_nc_h_lds(h_bytes));

  // every route's h row straight into LDS first (buffer_load ... lds, one
  // kilobyte per wave and piece; a wave whose piece lies past h issues none,
  // and lanes past the end of h read zeros into the padding up to the next
  // kilobyte), then the route positions and gate weights: all of it lands
  // before the weight rows issued next, whose loads stay in flight at the
  // barrier
  const auto rh = make_rsrc(p.h, h_bytes);
#pragma unroll
  for (int i = 0; i < kDcNcHLoads; ++i) {
    const uint32_t blk = (uint32_t)(i * kDcNcWaves + wave) * (kWave * 16);
    if (blk < h_bytes)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, s_dyn8 + blk, 16, blk + (uint32_t)lane * 16, 0, 0, 0);
  }
  const int rt = min(tid, R - 1);
  const int src_r = RS ? rt : p.route_src[rt];
  const float w_r = p.topk_w[rt];
  compiler_fence();

  int e_u[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int a = wave + u * kDcNcWaves;
    if constexpr (RS) e_u[u] = a < S ? min(max(sload(p.topk_idx, a), 0), p.E - 1) : -1;
    else e_u[u] = a < S ? slot_expert(p, a) : -1;
  }
  const uint32_t code_row = (uint32_t)p.I / 2, scale_row = (uint32_t)p.I / 16;
  // one resource spans all of W_down (and one its scales); the host checks
  // that their byte counts fit 31 bits
  const auto rd = make_rsrc(p.wd, (uint32_t)p.E * p.H * code_row);
  const auto rds = make_rsrc(p.sd, (uint32_t)p.E * p.H * scale_row);
  const int row = row0 + sub;
  const bool row_ok = row < p.H;
  uint4 cd[SLOTS][NC];
  uint32_t vd[SLOTS][NC];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const uint32_t r = (uint32_t)max(e_u[u], 0) * (uint32_t)p.H + (uint32_t)row;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      uint32_t oc, os;
      nc_chunk_offsets(sl, i, C, r * code_row, r * scale_row, row_ok && e_u[u] >= 0, oc, os);
      cd[u][i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rd, oc, 0, kStreamAux));
      vd[u][i] = __builtin_amdgcn_raw_buffer_load_b16(rds, os, 0, kStreamAux);
    }
  }
  compiler_fence();
  wait_vm<2 * SLOTS * NC>();                   // h, positions and weights have landed; the rows need not
  if (tid < R) {
    s_src[tid] = min(max(src_r, 0), R - 1);
    s_w[tid] = w_r;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  compiler_fence();
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    if (e_u[u] < 0) continue;
    int off = wave + u * kDcNcWaves, cnt = 1;   // route slots: the route itself
    if constexpr (!RS) expert_routes(p, e_u[u], off, cnt);
    const float gd = sload(p.gsc, e_u[u] * 3 + 2);
    for (int t = 0; t < cnt; ++t) {
      const int pos = off + t;
      const float one = opaque_one();
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        uint32_t hr[16];
        load_operand_chunk(s_h + (size_t)pos * p.I, min(sl + i * kNcLanes, C - 1), hr);
        acc = dot_chunk(cd[u][i], vd[u][i], hr, acc, one);
      }
      const float v = row16_sum(acc) * gd;
      if (sl == 0 && row_ok) s_o[s_src[pos] * rpw + sub] = v;
    }
  }
  __syncthreads();
  // y[t, row0 + r] = sum over slots j in order of w[t,j] * o[route (t,j), r]
  for (int i = tid; i < p.T * rpw; i += kDcNcThreads) {
    const int t = i / rpw, r = i - t * rpw;
    if (row0 + r >= p.H) continue;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j) acc = fmaf(s_w[t * p.k + j], s_o[(t * p.k + j) * rpw + r], acc);
    p.y[(size_t)t * p.H + row0 + r] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

// Chunks per lane of the multi-chunk kernels for rows of C chunks, or 0 when
// the one-chunk kernels take the row (C a power of two up to 64).
inline int nc_chunks(int C) {
  if (C <= 64 && (C & (C - 1)) == 0) return 0;
  const int nc = (C + kNcLanes - 1) / kNcLanes;
  return nc == 7 ? 8 : nc;                   // compiled for 1..6 and 8 (C <= 128)
}

void launch_gate_up_nc(int nc, const FfnParams& p, long long tasks, hipStream_t s) {
  const unsigned grid = (unsigned)std::max<long long>(1, tasks);
  switch (nc) {
    case 1: gate_up_nc_kernel<1><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 2: gate_up_nc_kernel<2><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 3: gate_up_nc_kernel<3><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 4: gate_up_nc_kernel<4><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 5: gate_up_nc_kernel<5><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 6: gate_up_nc_kernel<6><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    default: gate_up_nc_kernel<8><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
  }
}

void launch_down_nc(int nc, const FfnParams& p, long long tasks, hipStream_t s) {
  const unsigned grid = (unsigned)std::max<long long>(1, tasks);
  switch (nc) {
    case 1: down_nc_kernel<1><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 2: down_nc_kernel<2><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 3: down_nc_kernel<3><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 4: down_nc_kernel<4><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 5: down_nc_kernel<5><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    case 6: down_nc_kernel<6><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
    default: down_nc_kernel<8><<<grid, kThreads, 0, s>>>(p, (int)tasks); break;
  }
}

// Slots per wave of down_combine_nc_kernel for a batch's expert slots.
int dc_nc_slots_per_wave(long long slots) { return (int)((slots + kDcNcWaves - 1) / kDcNcWaves); }

// down_combine_nc_kernel<NC, S> with S = the slots per wave; only the
// instances with NC * S <= kDcNcMaxChunks exist (the policy sends no other
// batch here): false for any other.
template <int NC, bool RS, int S = 1>
bool launch_down_combine_nc_slots(const FfnParams& p, unsigned grid, size_t dyn, int per_wave, hipStream_t s) {
  if constexpr (NC * S > kDcNcMaxChunks) {
    return false;
  } else {
    if (per_wave == S) {
      down_combine_nc_kernel<NC, S, RS><<<grid, kDcNcThreads, dyn, s>>>(p);
      return true;
    }
    return launch_down_combine_nc_slots<NC, RS, S + 1>(p, grid, dyn, per_wave, s);
  }
}

// slots: expert slots (bucketed), or routes (RS: the small step's route slots)
template <bool RS = false>
bool launch_down_combine_nc(int nc, const FfnParams& p, unsigned grid, size_t dyn, int slots, hipStream_t s) {
  const int per_wave = dc_nc_slots_per_wave(slots);
  switch (nc) {
    case 1: return launch_down_combine_nc_slots<1, RS>(p, grid, dyn, per_wave, s);
    case 2: return launch_down_combine_nc_slots<2, RS>(p, grid, dyn, per_wave, s);
    case 3: return launch_down_combine_nc_slots<3, RS>(p, grid, dyn, per_wave, s);
    case 4: return launch_down_combine_nc_slots<4, RS>(p, grid, dyn, per_wave, s);
    case 5: return launch_down_combine_nc_slots<5, RS>(p, grid, dyn, per_wave, s);
    case 6: return launch_down_combine_nc_slots<6, RS>(p, grid, dyn, per_wave, s);
    case 8: return launch_down_combine_nc_slots<8, RS>(p, grid, dyn, per_wave, s);
    default: return false;
  }
}

// ------------------------------------------------------------------ host

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WorkspaceLayout {
  size_t h_off, o_off, plan_off, plan_down_off, rd_off, q_off, total;   // h [R, I] bf16, o [R, H] fp16, MFMA work plans (gate/up, down), row-dot list, unit counters
  int plan_max;
};

WorkspaceLayout workspace_layout(int T, int H, int I, int E, int k) {
  WorkspaceLayout L;
  const size_t R = (size_t)T * (size_t)k;
  L.h_off = 0;
  L.o_off = align256(R * (size_t)I * 2);
  L.plan_off = L.o_off + align256(R * (size_t)H * 2);
  // at most one partial chunk per expert slot plus R / kMmRoutes full ones;
  // the list has room for a multiple of 8 items (the MFMA grids' bound)
  L.plan_max = (int)(std::min<size_t>((size_t)E, R) + R / kMmRoutes);
  const size_t cap = ((size_t)L.plan_max + kXcds - 1) / kXcds * kXcds;
  L.plan_down_off = L.plan_off + align256((4 + 4 * cap) * 4);
  L.rd_off = L.plan_down_off + align256((4 + 4 * cap) * 4);
  // the row-dot list: its length and one expert per slot
  L.q_off = L.rd_off + align256((1 + std::min<size_t>((size_t)E, R)) * 4);
  L.total = L.q_off + align256((size_t)kWlQueueInts * 4);
  return L;
}

constexpr long long kMaxGrid = 1 << 20;   // one workgroup per task; the shape limits keep tasks below this
constexpr int kMfmaMinTokens = 64;      // batches from this size launch the MFMA kernels
constexpr int kRowPlanMinTokens = 16;   // batches above this size order the row-dot experts by count
constexpr int kMfmaMinRoutes = 16;      // experts with this many routes use them (standard weight layout)
constexpr int kMfmaMinRoutesPacked = 1; // with the packed copy: every expert of such a batch

// The streaming down kernel: K (= I) must run a multiple of four steps, at
// least eight, and the batch must hold enough routes for the items to
// outnumber the CU slots several times (with fewer, each workgroup takes one
// or two units and the claims and the pass-wise epilogue cost more than the
// streaming saves: measured at 2560 routes).
constexpr long long kStreamMinRoutes = 16384;
bool down_stream_fits(int I, long long R) {
  const int steps = I / kMmK;
  return I % kMmK == 0 && steps % kMmStages == 0 && steps >= 8 && R >= kStreamMinRoutes;
}

// Grid of the streaming down kernel: one workgroup per CU slot of the
// current device (compute units times the workgroups one holds, looked up
// once per device), at most one per unit, a multiple of the 8 classes; 0 when
// the device cannot be queried.
constexpr int kStreamMaxDevices = 64;
unsigned down_stream_grid(long long units) {
  static std::atomic<int> slots[kStreamMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStreamMaxDevices) return 0;
  int n = slots[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ffn_mfma_down_stream_kernel<2>, kMmThreads, 0) !=
            hipSuccess ||
        cus <= 0)
      return 0;
    n = cus * std::max(per_cu, 1);
    slots[dev].store(n, std::memory_order_relaxed);
  }
  const long long g = std::max<long long>(1, std::min<long long>(units, n));
  return (unsigned)((g + kXcds - 1) / kXcds * kXcds);
}

template <int LG>
void launch_gate_up(const FfnParams& p, long long tasks, hipStream_t s) {
  const unsigned grid = (unsigned)(std::max<long long>(1, tasks) + se_down_side_blocks(p.sr, kThreads / kWave));
  const int row_bytes = p.H * 2;
  const size_t x_lds = (size_t)std::max(1, std::min(kXStageBytes / row_bytes, 64)) * row_bytes;
  gate_up_kernel<LG><<<grid, kThreads, x_lds, s>>>(p, (int)tasks);
}

template <int LD>
void launch_down(const FfnParams& p, long long tasks, hipStream_t s) {
  const unsigned grid = (unsigned)std::max<long long>(1, tasks);
  down_kernel<LD><<<grid, kThreads, 0, s>>>(p, (int)tasks);
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_expert_ffn_workspace_size(int T, int H, int I, int E, int k) {
  if (T <= 0 || k <= 0 || H <= 0 || I <= 0 || E <= 0) return 0;
  return moe::workspace_layout(T, H, I, E, k).total;
}

namespace moe {

// Which kernels a call of these sizes launches (shared by expert_ffn and the
// work-list set-up of moe_step, so that both agree).
struct FfnPolicy {
  bool down_combine;   // fused down/unroute kernel (small batches)
  bool mfma;           // MFMA kernels launched
  int mfma_min;        // experts with at least this many routes take them (0: none)
  bool row_dots;       // row-dot kernels launched
  bool rd_plan;        // row-dot kernels read the sorted expert list
};

// Largest item count for which the MFMA work lists halve their route chunks:
// the items whose gate/up row tiles fill every compute unit twice (two
// workgroups per CU), within the list's capacity; 0 when no MFMA kernel runs.
int mfma_split_items(const FfnPolicy& f, int I, int plan_max) {
  if (!f.mfma) return 0;
  const int tiles_gu = (I + kMmRows - 1) / kMmRows;
  return std::min(plan_max, 2 * device_cu_count() / tiles_gu);
}

FfnPolicy ffn_policy(int T, int H, int I, int E, int k, bool packed) {
  FfnPolicy f;
  const long long R = (long long)T * k;
  const int lr_d = nc_chunks(I / 32) ? kNcLanes : lanes_per_row(I / 32);
  const size_t h_bytes = (size_t)R * I * 2;
  // one buffer resource spans all of W_down: its byte count must fit 31 bits
  const bool dc_fits = (size_t)E * H * (I / 2) < (size_t)0x7FFFFFFF;
  // h and o of the fused down/unroute kernel
  const size_t dc_lds = (nc_chunks(I / 32) ? dc_nc_h_lds((uint32_t)h_bytes) : h_bytes) + (size_t)R * (kWave / lr_d) * 4;
  // multi-chunk rows: the fused kernel holds nc chunks of each of its waves'
  // slots in registers, at most kDcNcMaxChunks of them
  const int nc_d = nc_chunks(I / 32);
  const long long dc_slots = std::min<long long>(E, R);
  const bool dc_regs = nc_d == 0 || nc_d * dc_nc_slots_per_wave(dc_slots) <= kDcNcMaxChunks;
  f.down_combine = R <= kDcMaxRoutes && dc_lds <= (size_t)kDcMaxLds && dc_fits && dc_regs;
  // Experts with many routes go to the MFMA kernels; only batches large
  // enough to have such experts (and not small enough for the fused
  // down/unroute kernel) launch them.  K (H for gate/up, I for down) must be a
  // multiple of the 64-wide step.  With the packed copy (one contiguous
  // kilobyte per weight load) the tiles beat one row-dot pass per route from
  // two routes on and match it at one (measured at decode_t256_zipf), so every
  // expert takes them and the row-dot kernels are not launched at all.
  f.mfma = !f.down_combine && T >= kMfmaMinTokens && H % kMmK == 0 && I % kMmK == 0;
  f.mfma_min = f.mfma ? (packed ? kMfmaMinRoutesPacked : kMfmaMinRoutes) : 0;
  f.row_dots = !f.mfma || f.mfma_min > 1;
  // above the small-batch size the row-dot kernels take their experts most
  // routes first from the list (their workgroups' lengths grow with the count)
  f.rd_plan = f.row_dots && T > kRowPlanMinTokens;
  return f;
}

bool ffn_work_lists(int T, int H, int I, int E, int k, bool packed, void* workspace, WorkLists* wl,
                    size_t* scratch_bytes) {
  if (T <= 0 || k < 1 || E < 1 || H < 32 || I < 32) return false;
  const FfnPolicy f = ffn_policy(T, H, I, E, k, packed);
  const WorkspaceLayout L = workspace_layout(T, H, I, E, k);
  char* ws = static_cast<char*>(workspace);
  wl->plan = reinterpret_cast<int32_t*>(ws + L.plan_off);
  wl->rd_list = reinterpret_cast<int32_t*>(ws + L.rd_off);
  wl->plan_max = L.plan_max;
  wl->mfma_min = f.mfma_min;
  wl->rd_plan = f.rd_plan ? 1 : 0;
  wl->queues = reinterpret_cast<int32_t*>(ws + L.q_off);
  wl->split_items = mfma_split_items(f, I, L.plan_max);
  wl->plan_down = reinterpret_cast<int32_t*>(ws + L.plan_down_off);
  *scratch_bytes = L.plan_off;
  return f.mfma || f.rd_plan;
}

moe_status expert_ffn(int stage, const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                      const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const float* g_scale, const float* topk_w, const int32_t* expert_count,
                      const int32_t* expert_offset, const int32_t* active_experts, const int32_t* n_active,
                      const int32_t* route_src, const int32_t* route_pos, const uint8_t* packed, int T, int H,
                      int I, int E, int k, void* workspace, size_t workspace_bytes, uint16_t* y, hipStream_t s,
                      bool lists_ready, const SharedRows* sr, bool* sr_done) {
  if (sr_done) *sr_done = false;
  if (stage < 1 || stage > 3) return MOE_ERR_INVALID_SHAPE;
  if (T < 0 || k < 1 || E < 1 || k > E || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32 || H > 4096 || I > 4096) return MOE_ERR_UNSUPPORTED;
  // the activations are read through one buffer resource (32-bit offsets)
  if ((long long)T * H * 2 >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  // rows of C = cols/32 chunks: one chunk per lane when C is a power of two
  // up to 64, else nc 16-lane passes (the multi-chunk kernels)
  const int nc_gu = nc_chunks(H / 32), nc_d = nc_chunks(I / 32);
  const int lr_gu = nc_gu ? kNcLanes : lanes_per_row(H / 32), lr_d = nc_d ? kNcLanes : lanes_per_row(I / 32);
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                        expert_offset, active_experts, n_active, route_src, route_pos, workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  if (packed && !aligned16(packed)) return MOE_ERR_MISALIGNED;
  const WorkspaceLayout L = workspace_layout(T, H, I, E, k);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  FfnParams p;
  p.x = x; p.wg = w_gate; p.sg = s_gate; p.wu = w_up; p.su = s_up; p.wd = w_down; p.sd = s_down;
  p.gsc = g_scale; p.topk_w = topk_w; p.count = expert_count; p.offset = expert_offset;
  p.active = active_experts; p.n_active_ptr = n_active; p.route_src = route_src; p.route_pos = route_pos;
  p.T = T; p.H = H; p.I = I; p.E = E; p.k = k;
  char* ws = static_cast<char*>(workspace);
  p.h = reinterpret_cast<uint16_t*>(ws + L.h_off);
  p.o = reinterpret_cast<uint16_t*>(ws + L.o_off);
  p.plan = reinterpret_cast<int32_t*>(ws + L.plan_off);
  p.plan_down = reinterpret_cast<int32_t*>(ws + L.plan_down_off);
  p.plan_max = L.plan_max;
  p.rd_list = reinterpret_cast<int32_t*>(ws + L.rd_off);
  p.queues = reinterpret_cast<int32_t*>(ws + L.q_off);
  p.y = y;
  p.sr = SharedRows{};
  p.lr_gu = lr_gu;
  p.lr_d = lr_d;
  p.packed = packed;
  // MFMA gate/up items per XCD that fill its compute units once
  {
    const int cus_per_xcd = device_cu_count() / kXcds;
    const int tiles_gu = (I + kMmRows - 1) / kMmRows;
    p.layer_items = (cus_per_xcd > 0 && cus_per_xcd % tiles_gu == 0) ? cus_per_xcd / tiles_gu : 0;
  }
  const long long R = (long long)T * k;
  const size_t h_bytes = (size_t)R * I * 2;
  const FfnPolicy pol = ffn_policy(T, H, I, E, k, packed != nullptr);
  const bool down_combine = pol.down_combine, mfma = pol.mfma, row_dots = pol.row_dots;
  p.mfma_min = pol.mfma_min;
  p.rd_plan = pol.rd_plan ? 1 : 0;
  p.split_items = mfma_split_items(pol, I, L.plan_max);

  const long long slots = std::min<long long>(E, (long long)T * k);
  const int rpt_gu = nc_gu ? kWavesPerBlock * kNcRowsPerWave : kWavesPerBlock * (kWave / lr_gu) * kGuUnits;
  const int rpt_d = nc_d ? kWavesPerBlock * kNcRowsPerWave : kWavesPerBlock * (kWave / lr_d) * kDUnits;
  const long long tasks_gu = slots * ((I + rpt_gu - 1) / rpt_gu);
  const long long tasks_d = slots * ((H + rpt_d - 1) / rpt_d);
  if (tasks_gu > kMaxGrid || tasks_d > kMaxGrid) return MOE_ERR_UNSUPPORTED;

  const long long items8 = ((long long)L.plan_max + kXcds - 1) / kXcds * kXcds;   // MFMA item bound, padded
  if ((mfma || p.rd_plan) && !lists_ready) {
    // the work lists (both stages use them; stage 2 alone rebuilds them)
    plan_kernel<<<1, kWlThreads, 0, s>>>(p);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  if (stage & 1) {
    if (row_dots) {
      if (nc_gu) {
        launch_gate_up_nc(nc_gu, p, tasks_gu, s);      // carries no shared-expert rows
      } else {
        p.sr = sr && sr->dn_nc > 0 ? *sr : SharedRows{};
        if (sr_done) *sr_done = p.sr.dn_nc > 0;
        if (lr_gu == 64) launch_gate_up<64>(p, tasks_gu, s);
        else launch_gate_up<0>(p, tasks_gu, s);
      }
      if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    }
    if (mfma) {
      const unsigned grid = (unsigned)(items8 * ((I + kMmRows - 1) / kMmRows));
      if (p.packed) ffn_mfma_kernel<true, true, 1><<<grid, kMmThreads, 0, s>>>(p);
      else ffn_mfma_kernel<true, false, 1><<<grid, kMmThreads, 0, s>>>(p);
      if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    }
  }
  if (!(stage & 2)) return MOE_OK;
  if (down_combine) {
    const int rpw = kWave / lr_d;
    const size_t dyn = (nc_d ? dc_nc_h_lds((uint32_t)h_bytes) : h_bytes) + (size_t)R * rpw * 4;
    const unsigned grid = (unsigned)((H + rpw - 1) / rpw);
    if (nc_d) {
      if (!launch_down_combine_nc(nc_d, p, grid, dyn, (int)slots, s)) return MOE_ERR_UNSUPPORTED;
    }
    else if (lr_d == 16) launch_down_combine<16>(p, grid, dyn, (int)slots, s);
    else launch_down_combine<0>(p, grid, dyn, (int)slots, s);
    return launch_status();
  }
  if (row_dots) {
    if (nc_d) launch_down_nc(nc_d, p, tasks_d, s);
    else if (lr_d == 16) launch_down<16>(p, tasks_d, s);
    else launch_down<0>(p, tasks_d, s);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  if (mfma) {
    if (p.packed) {
      // two row tiles per wave: each item's h rows are staged half as often
      // and every B fragment feeds two MFMAs
      const long long units = items8 * ((H + 2 * kMmRows - 1) / (2 * kMmRows));
      if (down_stream_fits(I, R)) {
        const unsigned grid = down_stream_grid(units);
        if (grid == 0) return MOE_ERR_HIP;
        ffn_mfma_down_stream_kernel<2><<<grid, kMmThreads, 0, s>>>(p, p.queues);
      } else {
        ffn_mfma_kernel<false, true, 2><<<(unsigned)units, kMmThreads, 0, s>>>(p);
      }
    } else {
      const unsigned grid = (unsigned)(items8 * ((H + kMmRows - 1) / kMmRows));
      ffn_mfma_kernel<false, false, 1><<<grid, kMmThreads, 0, s>>>(p);
    }
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  const long long cblocks = (long long)T * ((H + kCombineCols - 1) / kCombineCols);
  combine_kernel<<<(unsigned)cblocks, kThreads, 0, s>>>(p);
  return launch_status();
}

}  // namespace moe

extern "C" moe_status moe_expert_ffn_stage(int stage, const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                                           const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                                           const uint8_t* s_down, const float* g_scale, const float* topk_w,
                                           const int32_t* expert_count, const int32_t* expert_offset,
                                           const int32_t* active_experts, const int32_t* n_active,
                                           const int32_t* route_src, const int32_t* route_pos, int T, int H,
                                           int I, int E, int k, void* workspace, size_t workspace_bytes,
                                           uint16_t* y, void* stream) {
  return moe::expert_ffn(stage, x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                         expert_offset, active_experts, n_active, route_src, route_pos, nullptr, T, H, I, E, k,
                         workspace, workspace_bytes, y, static_cast<hipStream_t>(stream));
}

extern "C" moe_status moe_expert_ffn(const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                                     const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                                     const uint8_t* s_down, const float* g_scale, const float* topk_w,
                                     const int32_t* expert_count, const int32_t* expert_offset,
                                     const int32_t* active_experts, const int32_t* n_active,
                                     const int32_t* route_src, const int32_t* route_pos, int T, int H,
                                     int I, int E, int k, void* workspace, size_t workspace_bytes,
                                     uint16_t* y, void* stream) {
  return moe_expert_ffn_stage(3, x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                              expert_offset, active_experts, n_active, route_src, route_pos, T, H, I, E, k,
                              workspace, workspace_bytes, y, stream);
}

namespace moe {

// Batches up to this many routes take the small step (the selection and the
// routing outputs inside the gate/up launch, then the route-slot
// down/unroute);
// measured at the decode shape against routing + the expert kernels.
constexpr int kSmallStepMaxRoutes = kSgMaxRoutes;

bool small_step_ok(int T, int H, int I, int E, int k) {
  if (T < 1 || (long long)T * k > kSmallStepMaxRoutes) return false;
  if (k > 32) return false;
  // up to eight selection keys per lane: sixteen would take ~146 registers,
  // more than the gate/up workgroups (four per CU at least) may hold
  if (E > 8 * kWave) return false;
  // gate/up rows of one chunk per lane at H = 2048, or of several chunks per
  // lane (the row-dot kernels' one-chunk rows at other powers of two stay on
  // the three-kernel path)
  if (H != 64 * 32 && (nc_chunks(H / 32) == 0 || H * 2 > kSgNcXBytes)) return false;
  const int C = I / 32, nc_d = nc_chunks(C);
  if (nc_d == 0 && C > 64) return false;                          // down rows of one chunk per lane
  // the route-slot down/unroute holds nc_d chunks of every route slot of a
  // wave in registers
  if (nc_d > 0 && nc_d * dc_nc_slots_per_wave((long long)T * k) > kDcNcMaxChunks) return false;
  return ffn_policy(T, H, I, E, k, false).down_combine;
}

// nc = 0: rows of one chunk per lane (select_gate_up_kernel); else
// select_gate_up_nc_kernel<.., nc> (compiled for nc = 1..6 and 8)
template <int V, int KC>
void launch_select_gate_up(int nc, const FfnParams& p, const float* logits, const float* bias, int32_t* topk_idx,
                           float* topk_w, int tasks, int extra, hipStream_t s) {
  const unsigned grid = (unsigned)tasks + 1 + (unsigned)extra;
  switch (nc) {
    case 0: select_gate_up_kernel<V, KC><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 1: select_gate_up_nc_kernel<V, KC, 1><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 2: select_gate_up_nc_kernel<V, KC, 2><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 3: select_gate_up_nc_kernel<V, KC, 3><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 4: select_gate_up_nc_kernel<V, KC, 4><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 5: select_gate_up_nc_kernel<V, KC, 5><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    case 6: select_gate_up_nc_kernel<V, KC, 6><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
    default: select_gate_up_nc_kernel<V, KC, 8><<<grid, kThreads, 0, s>>>(p, logits, bias, topk_idx, topk_w, tasks); break;
  }
}

template <int V>
void launch_select_gate_up_k(int k, int nc, const FfnParams& p, const float* logits, const float* bias,
                             int32_t* topk_idx, float* topk_w, int tasks, int extra, hipStream_t s) {
  if (k == 10) launch_select_gate_up<V, 10>(nc, p, logits, bias, topk_idx, topk_w, tasks, extra, s);
  else launch_select_gate_up<V, 0>(nc, p, logits, bias, topk_idx, topk_w, tasks, extra, s);
}

// A shared expert's rows ride along in the small step (gate/up rows in the
// selection launch, down rows in the route-slot down/unroute) when the
// step's rows are of one chunk per lane (H = 2048), the shared rows of H =
// 2048 and Is = 512 or 1024, each down/unroute workgroup's rows fit its
// waves, and the shared h joins the LDS of the down/unroute.
bool small_step_side_ok(int T, int H, int I, int E, int k, const SharedRows& sr) {
  if (!small_step_ok(T, H, I, E, k) || H != 64 * 32 || nc_chunks(I / 32) != 0) return false;
  if (sr.gu_nc != 4 || (sr.dn_nc != 1 && sr.dn_nc != 2) || sr.T != T || sr.H != H) return false;
  const int R = T * k, rpw = kWave / lanes_per_row(I / 32);
  const size_t hs_bytes = (size_t)T * sr.Is * 2;
  return rpw <= kDcWaves && hs_bytes <= (size_t)kDcThreads * 16 &&
         dc_se_h_offset(R, I, rpw) + hs_bytes <= (size_t)kDcMaxLds;
}

moe_status small_step(const uint16_t* x, const float* logits, const float* bias, const uint8_t* w_gate,
                      const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                      const uint8_t* s_down, const float* g_scale, int T, int H, int I, int E, int k,
                      int32_t* topk_idx, float* topk_w, int32_t* expert_count, int32_t* expert_offset,
                      int32_t* active_experts, int32_t* n_active, int32_t* route_src, int32_t* route_pos,
                      void* workspace, uint16_t* y, hipStream_t s, int stage, const SharedRows* side) {
  const WorkspaceLayout L = workspace_layout(T, H, I, E, k);
  FfnParams p{};
  p.x = x; p.wg = w_gate; p.sg = s_gate; p.wu = w_up; p.su = s_up; p.wd = w_down; p.sd = s_down;
  p.gsc = g_scale; p.topk_w = topk_w; p.topk_idx = topk_idx;
  p.count = expert_count; p.offset = expert_offset; p.active = active_experts; p.n_active_ptr = n_active;
  p.route_src = route_src; p.route_pos = route_pos;
  p.T = T; p.H = H; p.I = I; p.E = E; p.k = k;
  char* ws = static_cast<char*>(workspace);
  p.h = reinterpret_cast<uint16_t*>(ws + L.h_off);
  p.o = reinterpret_cast<uint16_t*>(ws + L.o_off);
  p.y = y;
  p.sr = side ? *side : SharedRows{};       // the caller has checked small_step_side_ok
  const int nc_gu = H == 64 * 32 ? 0 : nc_chunks(H / 32), nc_d = nc_chunks(I / 32);
  p.lr_gu = nc_gu ? kNcLanes : 64;
  p.lr_d = nc_d ? kNcLanes : lanes_per_row(I / 32);
  const int R = T * k;
  // selection + gate/up: one workgroup per (route, 16 rows of I)
  static_assert(kWavesPerBlock * kGuUnits == kWavesPerBlock * kNcRowsPerWave, "16 rows of I per workgroup");
  const int tiles = (I + kWavesPerBlock * kGuUnits - 1) / (kWavesPerBlock * kGuUnits);
  const int tasks = R * tiles;                       // and one routing workgroup after them
  const int V = (E + kWave - 1) / kWave;
  // the shared expert's gate/up rows: one workgroup per four rows after the routing workgroup
  const int se_blocks = side ? (side->Is + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  if (stage & 1) {
    if (V <= 1) launch_select_gate_up_k<1>(k, nc_gu, p, logits, bias, topk_idx, topk_w, tasks, se_blocks, s);
    else if (V <= 2) launch_select_gate_up_k<2>(k, nc_gu, p, logits, bias, topk_idx, topk_w, tasks, se_blocks, s);
    else if (V <= 4) launch_select_gate_up_k<4>(k, nc_gu, p, logits, bias, topk_idx, topk_w, tasks, se_blocks, s);
    else launch_select_gate_up_k<8>(k, nc_gu, p, logits, bias, topk_idx, topk_w, tasks, se_blocks, s);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  if (!(stage & 2)) return MOE_OK;
  // route-slot down/unroute over rows of y
  const int rpw = kWave / p.lr_d;
  const size_t h_bytes = (size_t)R * I * 2;
  const size_t dyn = side ? dc_se_h_offset(R, I, rpw) + (size_t)T * side->Is * 2
                          : (nc_d ? dc_nc_h_lds((uint32_t)h_bytes) : h_bytes) + (size_t)R * rpw * 4;
  const unsigned grid = (unsigned)((H + rpw - 1) / rpw);
  if (nc_d) {
    if (!launch_down_combine_nc<true>(nc_d, p, grid, dyn, R, s)) return MOE_ERR_UNSUPPORTED;
  }
  else if (side && p.lr_d == 16) launch_down_combine<16, true, true>(p, grid, dyn, R, s);
  else if (side) launch_down_combine<0, true, true>(p, grid, dyn, R, s);
  else if (p.lr_d == 16) launch_down_combine<16, true>(p, grid, dyn, R, s);
  else launch_down_combine<0, true>(p, grid, dyn, R, s);
  return launch_status();
}

}  // namespace moe
