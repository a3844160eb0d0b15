// moe_expert_ffn_per_route: the routed experts without unique-expert reuse.
//
// The baseline of the reuse measurement on page "Persistent execution for
// Flash-Next GGUF on SM70" (section "Measurements that can accept or reject
// the design": the variants share the packed storage and the decoder; section
// "Opportunity sized from the actual routes": bytes issued per route against
// bytes of the distinct experts).  Every route (t, j) streams the weights of
// its expert e = topk_idx[t, j] itself, so an expert chosen by several tokens
// is read once per route; nothing is bucketed.  The per-route arithmetic is
// that of the reuse kernels: 16-byte chunks of e2m1 codes turned into exact
// bf16 pairs, v_dot2 products with the bf16 operand in fp32, one e4m3 scale
// per 16-value block, fixed-order lane sums, the fp32 global scale on the row
// total; h = bf16(SiLU(g) * u); each route's down output rounded once to fp16;
// y[t] = bf16(sum_j topk_w[t,j] * o[t*k + j]) in slot order.
//
// Kernels on one stream (the boundaries order the phases):
//   route_gate_up_kernel  (route, 16 rows of I): h[r, rows]
//   route_down_kernel     (route, 16 rows of H): o[r, rows]
//   route_combine_kernel  (token, 2048 columns): y
// A row is read by 16 lanes, lane l taking chunks l, l + 16, ... (NC of
// them); chunks past the row read as zero through the buffer range check.
#include "row_dot.h"

namespace moe {
namespace {

struct RouteParams {
  const uint16_t* x;
  const uint8_t *wg, *sg, *wu, *su, *wd, *sd;
  const float* gsc;
  const int32_t* topk_idx;
  const float* topk_w;
  int T, H, I, E, k;
  uint16_t* h;    // [R, I] bf16, row = flat route id t*k + j
  uint16_t* o;    // [R, H] fp16
  uint16_t* y;
};

constexpr int kPrLanes = 16;
constexpr int kPrRowsPerWave = kWave / kPrLanes;
constexpr int kPrRows = kWavesPerBlock * kPrRowsPerWave;     // rows per tile
constexpr uint32_t kPrOutOfRange = 0x80000000u;

typedef const __attribute__((address_space(4))) int32_t* pr_scalar_ptr;
typedef const __attribute__((address_space(4))) float* pr_scalar_fptr;

__device__ __forceinline__ uint32_t pr_f16(float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float pr_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// One row of C chunks: this lane's NC chunk loads (codes and the two scale
// bytes), offsets past the row or the matrix read zero.
template <int NC>
__device__ __forceinline__ void pr_load_row(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int row, bool row_ok,
                                            int C, uint32_t code_row, uint32_t scale_row, int sl, uint4 (&c)[NC],
                                            uint32_t (&v)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = sl + i * kPrLanes;
    const bool ok = row_ok && ch < C;
    const uint32_t oc = ok ? (uint32_t)row * code_row + (uint32_t)ch * 16u : kPrOutOfRange;
    const uint32_t os = ok ? (uint32_t)row * scale_row + (uint32_t)ch * 2u : kPrOutOfRange;
    c[i] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, kStreamAux));
    v[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, kStreamAux);
  }
}

template <int NC>
__global__ __launch_bounds__(kThreads, 2) void route_gate_up_kernel(RouteParams p, int tiles) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / kPrLanes, sl = lane & (kPrLanes - 1);
  const int r = blockIdx.x / tiles, tile = blockIdx.x - r * tiles;
  const int e = min(max(((pr_scalar_ptr)p.topk_idx)[r], 0), p.E - 1);
  const int t = r / p.k;
  const int C = p.H / 32;
  const uint32_t code_row = (uint32_t)p.H / 2, scale_row = (uint32_t)p.H / 16;
  const uint32_t mat_codes = (uint32_t)p.I * code_row, mat_scales = (uint32_t)p.I * scale_row;
  const int row = tile * kPrRows + wave * kPrRowsPerWave + sub;
  const bool row_ok = row < p.I;
  uint4 cg[NC], cu[NC];
  uint32_t vg[NC], vu[NC];
  pr_load_row<NC>(make_rsrc(p.wg + (size_t)e * mat_codes, mat_codes), make_rsrc(p.sg + (size_t)e * mat_scales, mat_scales),
                  row, row_ok, C, code_row, scale_row, sl, cg, vg);
  pr_load_row<NC>(make_rsrc(p.wu + (size_t)e * mat_codes, mat_codes), make_rsrc(p.su + (size_t)e * mat_scales, mat_scales),
                  row, row_ok, C, code_row, scale_row, sl, cu, vu);
  const float Gg = ((pr_scalar_fptr)p.gsc)[e * 3 + 0], Gu = ((pr_scalar_fptr)p.gsc)[e * 3 + 1];
  const uint16_t* xrow = p.x + (size_t)t * p.H;
  const float one = opaque_one();
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t xr[16];
    load_operand_chunk(xrow, min(sl + i * kPrLanes, C - 1), xr);
    ag = dot_chunk(cg[i], vg[i], xr, ag, one);
    au = dot_chunk(cu[i], vu[i], xr, au, one);
  }
  const float gs = row16_sum(ag) * Gg, us = row16_sum(au) * Gu;
  if (sl == 0 && row_ok) p.h[(size_t)r * p.I + row] = (uint16_t)f32_to_bf16_rne(silu(gs) * us);
}

template <int NC>
__global__ __launch_bounds__(kThreads, 2) void route_down_kernel(RouteParams p, int tiles) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / kPrLanes, sl = lane & (kPrLanes - 1);
  const int r = blockIdx.x / tiles, tile = blockIdx.x - r * tiles;
  const int e = min(max(((pr_scalar_ptr)p.topk_idx)[r], 0), p.E - 1);
  const int C = p.I / 32;
  const uint32_t code_row = (uint32_t)p.I / 2, scale_row = (uint32_t)p.I / 16;
  const uint32_t mat_codes = (uint32_t)p.H * code_row, mat_scales = (uint32_t)p.H * scale_row;
  const int row = tile * kPrRows + wave * kPrRowsPerWave + sub;
  const bool row_ok = row < p.H;
  uint4 cd[NC];
  uint32_t vd[NC];
  pr_load_row<NC>(make_rsrc(p.wd + (size_t)e * mat_codes, mat_codes), make_rsrc(p.sd + (size_t)e * mat_scales, mat_scales),
                  row, row_ok, C, code_row, scale_row, sl, cd, vd);
  const float Gd = ((pr_scalar_fptr)p.gsc)[e * 3 + 2];
  const uint16_t* hrow = p.h + (size_t)r * p.I;
  const float one = opaque_one();
  float ad = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    uint32_t hr[16];
    load_operand_chunk(hrow, min(sl + i * kPrLanes, C - 1), hr);
    ad = dot_chunk(cd[i], vd[i], hr, ad, one);
  }
  const float v = row16_sum(ad) * Gd;
  if (sl == 0 && row_ok) p.o[(size_t)r * p.H + row] = (uint16_t)pr_f16(v);
}

constexpr int kPrCombineCols = 8 * kThreads;
constexpr int kPrMaxK = 32;

// y[t, c..c+7] = bf16(sum over j in slot order of w[t,j] * o[t*k + j, c..c+7]).
__global__ __launch_bounds__(kThreads) void route_combine_kernel(RouteParams p) {
  const int col_blocks = (p.H + kPrCombineCols - 1) / kPrCombineCols;
  const int t = blockIdx.x / col_blocks;
  const int c = (blockIdx.x - t * col_blocks) * kPrCombineCols + 8 * threadIdx.x;
  if (c >= p.H) return;                        // H is a multiple of 32: c + 8 <= H
  uint4 ov[kPrMaxK];
#pragma unroll
  for (int j = 0; j < kPrMaxK; ++j)
    if (j < p.k) ov[j] = *reinterpret_cast<const uint4*>(p.o + ((size_t)t * p.k + j) * p.H + c);
  float yv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kPrMaxK; ++j) {
    if (j < p.k) {
      const float w = ((pr_scalar_fptr)p.topk_w)[t * p.k + j];
      const uint32_t d[4] = {ov[j].x, ov[j].y, ov[j].z, ov[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yv[2 * q] = fmaf(w, pr_f32(d[q] & 0xFFFFu), yv[2 * q]);
        yv[2 * q + 1] = fmaf(w, pr_f32(d[q] >> 16), yv[2 * q + 1]);
      }
    }
  }
  uint32_t yb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) yb[q] = f32_to_bf16_rne(yv[2 * q]) | (f32_to_bf16_rne(yv[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(p.y + (size_t)t * p.H + c) = make_uint4(yb[0], yb[1], yb[2], yb[3]);
}

template <int NC>
void pr_launch(const RouteParams& p, unsigned tiles_gu, unsigned tiles_d, int R, hipStream_t s, int stage) {
  if (stage == 1) route_gate_up_kernel<NC><<<(unsigned)R * tiles_gu, kThreads, 0, s>>>(p, (int)tiles_gu);
  else route_down_kernel<NC><<<(unsigned)R * tiles_d, kThreads, 0, s>>>(p, (int)tiles_d);
}

template <int... NCS>
void pr_dispatch(int nc, const RouteParams& p, unsigned tiles_gu, unsigned tiles_d, int R, hipStream_t s, int stage) {
  ((nc == NCS ? (pr_launch<NCS>(p, tiles_gu, tiles_d, R, s, stage), 0) : 0), ...);
}

inline size_t pr_align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace
}  // namespace moe

extern "C" moe_status moe_expert_ffn_per_route(const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                                               const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                                               const uint8_t* s_down, const float* g_scale, const int32_t* topk_idx,
                                               const float* topk_w, int T, int H, int I, int E, int k,
                                               void* workspace, size_t workspace_bytes, uint16_t* y, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || E < 1 || k > E || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32 || H > 4096 || I > 4096) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)T * k;
  const unsigned tiles_gu = (unsigned)((I + kPrRows - 1) / kPrRows), tiles_d = (unsigned)((H + kPrRows - 1) / kPrRows);
  if (R * tiles_gu >= (1ll << 31) || R * tiles_d >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_idx, topk_w, workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  // h [R, I] bf16 then o [R, H] fp16: within moe_expert_ffn_workspace_size
  const size_t h_bytes = pr_align256((size_t)R * I * 2), need = h_bytes + pr_align256((size_t)R * H * 2);
  if (workspace_bytes < need || workspace_bytes < moe_expert_ffn_workspace_size(T, H, I, E, k))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  RouteParams p;
  p.x = x; p.wg = w_gate; p.sg = s_gate; p.wu = w_up; p.su = s_up; p.wd = w_down; p.sd = s_down;
  p.gsc = g_scale; p.topk_idx = topk_idx; p.topk_w = topk_w;
  p.T = T; p.H = H; p.I = I; p.E = E; p.k = k;
  p.h = static_cast<uint16_t*>(workspace);
  p.o = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + h_bytes);
  p.y = y;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // chunks per lane: 1..8 for rows of 32..4096 values (checked above)
  const int nc_gu = (H / 32 + kPrLanes - 1) / kPrLanes, nc_d = (I / 32 + kPrLanes - 1) / kPrLanes;
  pr_dispatch<1, 2, 3, 4, 5, 6, 7, 8>(nc_gu, p, tiles_gu, tiles_d, (int)R, s, 1);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  pr_dispatch<1, 2, 3, 4, 5, 6, 7, 8>(nc_d, p, tiles_gu, tiles_d, (int)R, s, 2);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const unsigned cblocks = (unsigned)(T * ((H + kPrCombineCols - 1) / kPrCombineCols));
  route_combine_kernel<<<cblocks, kThreads, 0, s>>>(p);
  return launch_status();
}
