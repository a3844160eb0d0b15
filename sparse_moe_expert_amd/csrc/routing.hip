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
// same page paragraph describes one workgroup doing all of it for batches of
// up to 64 tokens; moe_route_bucket does that here.
//
// Selection (gfx950): one 64-lane wavefront per token.  Lane l holds experts
// [l*V, l*V+V) as 32-bit keys ordered(z), an unsigned integer with the same
// order as the fp32 score (-0.0 first canonicalised to +0.0); absent experts
// hold 0, below every real key.  Each of the k rounds takes the wave maximum
// of the lanes' best keys (DPP row steps, then the four row maxima as
// scalars), then the lowest lane holding that key (ballot): lanes own
// ascending id ranges, so that lane - and its first matching slot - has the
// lowest id among equal scores.  Only the winning lane recomputes its best.
//
// Bucketing (one 1024-thread workgroup): LDS histogram of expert ids
// (integer atomics: counts do not depend on their order), block-wide
// exclusive scans of the counts and of the "count > 0" flags, then a stable
// scatter in chunks of 1024 routes: lanes of a wavefront with the same expert
// are found with one ballot per id bit; rank among them + counts of earlier
// wavefronts in the chunk + the expert's running base gives the position.
// Positions never depend on timing, so the result is exact and reproducible.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / kWave;
constexpr int kFusedMaxTokens = 64;        // one workgroup routes and buckets up to this many tokens
constexpr int kFusedMaxRoutes = 2048;

__device__ __forceinline__ uint32_t ordered_bits(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0;                 // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the wavefront (wave-uniform result).  DPP steps reduce each
// 16-lane row; the four row results are then read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124>(v));   // row_ror:4
  v = max(v, dpp_u32<0x128>(v));   // row_ror:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum over the wavefront in a fixed order (wave-uniform result).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Top-k of one token's row: idx/weights of slot j end up in lane j.
template <int V>
__device__ __forceinline__ void select_token(const float* __restrict__ row, const float* __restrict__ bias, int E,
                                             int k, int lane, int& my_e, float& my_w) {
  const int e0 = lane * V;
  float zv[V];
  const bool full = (V % 4 == 0) && (E % 4 == 0) && (e0 + V <= E);
  if (full) {                                   // 16-byte vector loads
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const float4 l4 = *reinterpret_cast<const float4*>(row + e0 + i);
      zv[i] = l4.x; zv[i + 1] = l4.y; zv[i + 2] = l4.z; zv[i + 3] = l4.w;
      if (bias) {
        const float4 b4 = *reinterpret_cast<const float4*>(bias + e0 + i);
        zv[i] += b4.x; zv[i + 1] += b4.y; zv[i + 2] += b4.z; zv[i + 3] += b4.w;  // fp32 adds, RNE
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = e0 + i;
      zv[i] = 0.0f;
      if (e < E) zv[i] = bias ? row[e] + bias[e] : row[e];
    }
  }
  uint32_t key[V];
  uint32_t best = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    key[i] = (e0 + i < E) ? ordered_bits(zv[i]) : 0u;
    best = max(best, key[i]);
  }
  uint32_t my_key = 0, key0 = 0;
  my_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t wbest = wave_max_u32(best);
    const uint64_t holders = __ballot(best == wbest);
    const int wl = __builtin_ctzll(holders);    // lowest lane: lowest ids
    int pick = 0;
    if (lane == wl) {
      int first = V;
#pragma unroll
      for (int i = V - 1; i >= 0; --i)
        if (key[i] == wbest) first = i;
      pick = e0 + first;
      uint32_t nb = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (i == first) key[i] = 0;             // retire the winner
        nb = max(nb, key[i]);
      }
      best = nb;
    }
    const int e_sel = __builtin_amdgcn_readlane(pick, wl);
    if (j == 0) key0 = wbest;
    if (lane == j) { my_key = wbest; my_e = e_sel; }
  }
  // Renormalised softmax over the chosen set: w_j = exp(z_j - z_0) / sum.
  const float z0 = from_ordered(key0);
  const float pj = (lane < k) ? __builtin_expf(from_ordered(my_key) - z0) : 0.0f;
  my_w = pj / wave_sum_f32(pj);
}

template <int V>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                           // whole wavefront leaves together
  int e;
  float w;
  select_token<V>(logits + (size_t)t * E, bias, E, k, lane, e, w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = e;
    topk_w[(size_t)t * k + lane] = w;
  }
}

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
};

// Bucket R routes whose expert ids are ids[0..R) (global or LDS).
__device__ __forceinline__ void bucket_block(const int32_t* ids, int R, int E, int id_bits, BucketShared& sh,
                                             int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
                                             int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
                                             int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int e = tid; e < 1024; e += kBucketThreads) sh.base[e] = 0;
  for (int i = tid; i < kBucketWaves * 1024; i += kBucketThreads) (&sh.wcnt[0][0])[i] = 0;
  __syncthreads();
  // ids outside [0, E) violate the precondition; clamping keeps every access
  // in bounds
  for (int r = tid; r < R; r += kBucketThreads) atomicAdd(&sh.base[min(max(ids[r], 0), E - 1)], 1);
  __syncthreads();

  // scans (E <= 1024: one expert per thread)
  const int c = tid < E ? sh.base[tid] : 0;
  int total_routes, total_active;
  const int off = block_exclusive_scan(c, sh.wave_tot, &total_routes);
  const int apos = block_exclusive_scan(c > 0 ? 1 : 0, sh.wave_tot, &total_active);
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
  __syncthreads();

  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < R; c0 += kBucketThreads) {
    const int r = c0 + tid;
    const bool valid = r < R;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
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
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&sh.base[e], wcount);
      sh.wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBucketThreads) void bucket_routes_kernel(
    const int32_t* __restrict__ topk_idx, int R, int E, int id_bits,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  __shared__ BucketShared sh;
  bucket_block(topk_idx, R, E, id_bits, sh, expert_count, expert_offset, active_experts, n_active, route_src,
               route_pos);
}

// Route and bucket a small batch in one workgroup: wavefront w selects for
// tokens w, w+16, ...; the ids stay in LDS for the bucketing.
template <int V>
__global__ __launch_bounds__(kBucketThreads) void route_bucket_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k, int id_bits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ active_experts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ route_src, int32_t* __restrict__ route_pos) {
  __shared__ BucketShared sh;
  __shared__ int s_ids[kFusedMaxRoutes];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kBucketWaves) {
    int e;
    float w;
    select_token<V>(logits + (size_t)t * E, bias, E, k, lane, e, w);
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = e;
      topk_w[(size_t)t * k + lane] = w;
      s_ids[t * k + lane] = e;
    }
  }
  __syncthreads();
  bucket_block(s_ids, T * k, E, id_bits, sh, expert_count, expert_offset, active_experts, n_active, route_src,
               route_pos);
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
  if (V <= 1) route_topk_kernel<1><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 2) route_topk_kernel<2><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 4) route_topk_kernel<4><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else if (V <= 8) route_topk_kernel<8><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
  else route_topk_kernel<16><<<grid, block, 0, s>>>(logits, bias, T, E, k, topk_idx, topk_w);
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
      topk_idx, T * k, E, id_bits_for(E), expert_count, expert_offset, active_experts, n_active, route_src,
      route_pos);
  return launch_status();
}

extern "C" moe_status moe_route_bucket(const float* logits, const float* bias, int T, int E, int k,
                                       int32_t* topk_idx, float* topk_w,
                                       int32_t* expert_count, int32_t* expert_offset,
                                       int32_t* active_experts, int32_t* n_active,
                                       int32_t* route_src, int32_t* route_pos, void* stream) {
  using namespace moe;
  moe_status st = check_route_args(logits, bias, T, E, k, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  st = check_bucket_args(T, E, k, expert_count, expert_offset, active_experts, n_active, route_src, route_pos);
  if (st != MOE_OK || T == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int bits = id_bits_for(E);
  if (T <= kFusedMaxTokens && T * k <= kFusedMaxRoutes) {
    const int V = (E + kWave - 1) / kWave;
#define MOE_RB(VV)                                                                                          \
  route_bucket_kernel<VV><<<1, kBucketThreads, 0, s>>>(logits, bias, T, E, k, bits, topk_idx, topk_w,       \
                                                        expert_count, expert_offset, active_experts, n_active, \
                                                        route_src, route_pos)
    if (V <= 1) MOE_RB(1);
    else if (V <= 2) MOE_RB(2);
    else if (V <= 4) MOE_RB(4);
    else if (V <= 8) MOE_RB(8);
    else MOE_RB(16);
#undef MOE_RB
    return launch_status();
  }
  launch_route(logits, bias, T, E, k, topk_idx, topk_w, s);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bucket_routes_kernel<<<1, kBucketThreads, 0, s>>>(topk_idx, T * k, E, bits, expert_count, expert_offset,
                                                     active_experts, n_active, route_src, route_pos);
  return launch_status();
}
