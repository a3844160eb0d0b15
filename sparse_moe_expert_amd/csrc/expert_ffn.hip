// moe_expert_ffn: routed NVFP4 SwiGLU experts with a weighted, fixed-order unroute.
//
// The chain of the SM70 design note (page "Persistent execution for Flash-Next
// GGUF on SM70", sections "What the measurements establish" and "First
// implementation boundary"): gate/up fused with SiLU * multiply, then down,
// then the weighted unroute with routes summed in a fixed order rather than
// by arrival-ordered floating-point atomics.  Unique-expert reuse: a task owns
// (active expert, row tile) and streams those weight rows from HBM once for
// all of the expert's routes (the page's first boundary, step 2; the b12x
// kernel's cost is "weight bytes" of the unique experts - page "Qwen3.8 Flash
// Next on LiL/vLLM", section "11.13 Where the decode step's time actually
// goes").
//
// Kernels (one stream, no host sync):
//   gate_up_gemv  task = (active expert a, tile of I rows).  Lane groups of Lr
//                 lanes share a row; each lane reads 16-byte chunks of codes
//                 (32 e2m1 values), converts byte pairs to bf16 with
//                 v_cvt_scalef32_pk_bf16_fp4 (exact), takes v_dot2 products
//                 with the token's bf16 activations held in registers, applies
//                 one e4m3 scale per 16 values, then a butterfly sum over the
//                 Lr lanes.  Epilogue: SiLU(g) * u, rounded to bf16 into h[route].
//   down_gemv     task = (active expert a, tile of H rows): same structure with
//                 h as the operand; o[route, row] = fp32 result.
//   combine       y[t] = bf16( sum_{j=0}^{k-1} w[t,j] * o[route_pos[t*k+j]] )
//                 in slot order.
// Tokens of an expert are taken NT at a time (NT <= 4 held in registers);
// experts with more routes loop over token groups, re-reading their weight
// rows from L2.
#include <algorithm>

#include "moe_common.h"

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
  const int32_t* count;
  const int32_t* offset;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* route_src;
  const int32_t* route_pos;
  int T, H, I, E, k;
  uint16_t* h;   // workspace: [R, I] bf16, row = bucket position
  float* o;      // workspace: [R, H] fp32, row = bucket position
  uint16_t* y;
  int lr_gu;     // lanes per gate/up row (power of two, <= 64)
  int lr_d;      // lanes per down row
};

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kNtMax = 4;

// One 16-byte chunk (32 NVFP4 values, two scale blocks) dotted with NT
// operand vectors.  xr[t][i] holds operand elements 2i, 2i+1 of the chunk as
// bf16x2.  acc gets sum * 2^-8 (see e4m3_to_f32_div256).
template <int NT>
__device__ __forceinline__ void dot_chunk(const uint4 codes, uint32_t s2,
                                          const uint32_t (&xr)[NT][16], float (&acc)[NT]) {
  const float s0 = e4m3_to_f32_div256(s2 & 0xFFu);
  const float s1 = e4m3_to_f32_div256((s2 >> 8) & 0xFFu);
  bf16x2 w[16];
  w[0] = fp4x2_to_bf16x2<0>(codes.x);  w[1] = fp4x2_to_bf16x2<1>(codes.x);
  w[2] = fp4x2_to_bf16x2<2>(codes.x);  w[3] = fp4x2_to_bf16x2<3>(codes.x);
  w[4] = fp4x2_to_bf16x2<0>(codes.y);  w[5] = fp4x2_to_bf16x2<1>(codes.y);
  w[6] = fp4x2_to_bf16x2<2>(codes.y);  w[7] = fp4x2_to_bf16x2<3>(codes.y);
  w[8] = fp4x2_to_bf16x2<0>(codes.z);  w[9] = fp4x2_to_bf16x2<1>(codes.z);
  w[10] = fp4x2_to_bf16x2<2>(codes.z); w[11] = fp4x2_to_bf16x2<3>(codes.z);
  w[12] = fp4x2_to_bf16x2<0>(codes.w); w[13] = fp4x2_to_bf16x2<1>(codes.w);
  w[14] = fp4x2_to_bf16x2<2>(codes.w); w[15] = fp4x2_to_bf16x2<3>(codes.w);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) p0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xr[t][i]), p0, false);
#pragma unroll
    for (int i = 8; i < 16; ++i) p1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xr[t][i]), p1, false);
    acc[t] = fmaf(p0, s0, acc[t]);
    acc[t] = fmaf(p1, s1, acc[t]);
  }
}

// Load the 64-byte operand chunk `chunk` of a bf16 row into xr (16 dwords).
__device__ __forceinline__ void load_operand_chunk(const uint16_t* row, int chunk, uint32_t (&dst)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(row + (size_t)chunk * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    dst[4 * q + 0] = v.x; dst[4 * q + 1] = v.y; dst[4 * q + 2] = v.z; dst[4 * q + 3] = v.w;
  }
}

// Expert id, route count and first bucket position of active slot a.  The
// values come from moe_bucket_routes; they are clamped into range so that
// inputs violating that precondition give wrong results, never out-of-bounds
// accesses.
__device__ __forceinline__ void expert_routes(const FfnParams& p, int a, int& e, int& cnt, int& off) {
  const int R = p.T * p.k;
  e = min(max(p.active[a], 0), p.E - 1);
  off = min(max(p.offset[e], 0), R);
  cnt = min(max(p.count[e], 0), R - off);
}

// ------------------------------------------------------------------ gate/up

template <int CPL, int U, int NT>
__device__ __forceinline__ void gate_up_rows(const FfnParams& p, int e, int first_pos, int tile,
                                             int rows_per_task, int Lr, int sub, int sl, int wave) {
  const int rpw = kWave / Lr;
  const size_t code_row = (size_t)p.H / 2, scale_row = (size_t)p.H / 16;
  const uint8_t* wg = p.wg + (size_t)e * p.I * code_row;
  const uint8_t* wu = p.wu + (size_t)e * p.I * code_row;
  const uint8_t* sg = p.sg + (size_t)e * p.I * scale_row;
  const uint8_t* su = p.su + (size_t)e * p.I * scale_row;

  uint32_t xr[CPL][NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = min(max(p.route_src[first_pos + t] / p.k, 0), p.T - 1);
    const uint16_t* xrow = p.x + (size_t)tok * p.H;
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_operand_chunk(xrow, c * Lr + sl, xr[c][t]);
  }

  int rows[U];
  uint4 cg[U][CPL], cu[U][CPL];
  uint32_t vg[U][CPL], vu[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    rows[u] = tile * rows_per_task + u * (kWavesPerBlock * rpw) + wave * rpw + sub;
    const bool ok = rows[u] < p.I;
    const size_t r = ok ? (size_t)rows[u] : 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int chunk = c * Lr + sl;
      cg[u][c] = ok ? *reinterpret_cast<const uint4*>(wg + r * code_row + (size_t)chunk * 16) : make_uint4(0, 0, 0, 0);
      cu[u][c] = ok ? *reinterpret_cast<const uint4*>(wu + r * code_row + (size_t)chunk * 16) : make_uint4(0, 0, 0, 0);
      vg[u][c] = ok ? *reinterpret_cast<const uint16_t*>(sg + r * scale_row + (size_t)chunk * 2) : 0u;
      vu[u][c] = ok ? *reinterpret_cast<const uint16_t*>(su + r * scale_row + (size_t)chunk * 2) : 0u;
    }
  }

  float ag[U][NT], au[U][NT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[u][t] = au[u][t] = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      dot_chunk<NT>(cg[u][c], vg[u][c], xr[c], ag[u]);
      dot_chunk<NT>(cu[u][c], vu[u][c], xr[c], au[u]);
    }

  const float Gg = p.gsc[e * 3 + 0] * 256.0f, Gu = p.gsc[e * 3 + 1] * 256.0f;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float g = group_sum(ag[u][t], Lr) * Gg;
      const float v = group_sum(au[u][t], Lr) * Gu;
      if (sl == t % Lr && rows[u] < p.I)   // one lane per (token, row) stores
        p.h[(size_t)(first_pos + t) * p.I + rows[u]] = (uint16_t)f32_to_bf16_rne(silu(g) * v);
    }
}

template <int CPL, int U>
__global__ __launch_bounds__(kThreads) void gate_up_gemv(FfnParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int Lr = p.lr_gu, rpw = kWave / Lr;
  const int sub = lane / Lr, sl = lane & (Lr - 1);
  const int rows_per_task = kWavesPerBlock * rpw * U;
  const int tiles = (p.I + rows_per_task - 1) / rows_per_task;
  const int total = min(max(*p.n_active, 0), p.E) * tiles;
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int a = task / tiles, tile = task - a * tiles;
    int e, cnt, off;
    expert_routes(p, a, e, cnt, off);
    for (int tg = 0; tg < cnt; tg += kNtMax) {
      const int nt = min(kNtMax, cnt - tg);
      if (nt == 1) gate_up_rows<CPL, U, 1>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else if (nt == 2) gate_up_rows<CPL, U, 2>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else if (nt == 3) gate_up_rows<CPL, U, 3>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else gate_up_rows<CPL, U, 4>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
    }
  }
}

// ------------------------------------------------------------------ down

template <int CPL, int U, int NT>
__device__ __forceinline__ void down_rows(const FfnParams& p, int e, int first_pos, int tile,
                                          int rows_per_task, int Lr, int sub, int sl, int wave) {
  const int rpw = kWave / Lr;
  const size_t code_row = (size_t)p.I / 2, scale_row = (size_t)p.I / 16;
  const uint8_t* wd = p.wd + (size_t)e * p.H * code_row;
  const uint8_t* sd = p.sd + (size_t)e * p.H * scale_row;

  uint32_t hr[CPL][NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint16_t* hrow = p.h + (size_t)(first_pos + t) * p.I;
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_operand_chunk(hrow, c * Lr + sl, hr[c][t]);
  }

  int rows[U];
  uint4 cd[U][CPL];
  uint32_t vd[U][CPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    rows[u] = tile * rows_per_task + u * (kWavesPerBlock * rpw) + wave * rpw + sub;
    const bool ok = rows[u] < p.H;
    const size_t r = ok ? (size_t)rows[u] : 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int chunk = c * Lr + sl;
      cd[u][c] = ok ? *reinterpret_cast<const uint4*>(wd + r * code_row + (size_t)chunk * 16) : make_uint4(0, 0, 0, 0);
      vd[u][c] = ok ? *reinterpret_cast<const uint16_t*>(sd + r * scale_row + (size_t)chunk * 2) : 0u;
    }
  }

  float ad[U][NT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) ad[u][t] = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < CPL; ++c) dot_chunk<NT>(cd[u][c], vd[u][c], hr[c], ad[u]);

  const float Gd = p.gsc[e * 3 + 2] * 256.0f;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = group_sum(ad[u][t], Lr) * Gd;
      if (sl == t % Lr && rows[u] < p.H) p.o[(size_t)(first_pos + t) * p.H + rows[u]] = v;
    }
}

template <int CPL, int U>
__global__ __launch_bounds__(kThreads) void down_gemv(FfnParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int Lr = p.lr_d, rpw = kWave / Lr;
  const int sub = lane / Lr, sl = lane & (Lr - 1);
  const int rows_per_task = kWavesPerBlock * rpw * U;
  const int tiles = (p.H + rows_per_task - 1) / rows_per_task;
  const int total = min(max(*p.n_active, 0), p.E) * tiles;
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int a = task / tiles, tile = task - a * tiles;
    int e, cnt, off;
    expert_routes(p, a, e, cnt, off);
    for (int tg = 0; tg < cnt; tg += kNtMax) {
      const int nt = min(kNtMax, cnt - tg);
      if (nt == 1) down_rows<CPL, U, 1>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else if (nt == 2) down_rows<CPL, U, 2>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else if (nt == 3) down_rows<CPL, U, 3>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
      else down_rows<CPL, U, 4>(p, e, off + tg, tile, rows_per_task, Lr, sub, sl, wave);
    }
  }
}

// ------------------------------------------------------------------ combine

__global__ __launch_bounds__(kThreads) void combine_kernel(FfnParams p) {
  const int pairs = p.H / 2;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (long long)p.T * pairs) return;
  const int t = (int)(gid / pairs);
  const int c = (int)(gid - (long long)t * pairs) * 2;
  float y0 = 0.0f, y1 = 0.0f;
  for (int j = 0; j < p.k; ++j) {                 // slot order: fixed
    const float w = p.topk_w[(size_t)t * p.k + j];
    const int pos = min(max(p.route_pos[(size_t)t * p.k + j], 0), p.T * p.k - 1);
    const float2 ov = *reinterpret_cast<const float2*>(p.o + (size_t)pos * p.H + c);
    y0 = fmaf(w, ov.x, y0);
    y1 = fmaf(w, ov.y, y1);
  }
  reinterpret_cast<uint32_t*>(p.y)[((size_t)t * p.H + c) >> 1] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
}

constexpr int kU = 4;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WorkspaceLayout {
  size_t h_off, o_off, total;
};

WorkspaceLayout workspace_layout(int T, int H, int I, int k) {
  WorkspaceLayout L;
  const size_t R = (size_t)T * (size_t)k;
  L.h_off = 0;
  L.o_off = align256(R * (size_t)I * 2);
  L.total = L.o_off + align256(R * (size_t)H * 4) + 256;   // + control region
  return L;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_expert_ffn_workspace_size(int T, int H, int I, int E, int k) {
  (void)E;
  if (T <= 0 || k <= 0 || H <= 0 || I <= 0) return 0;
  return moe::workspace_layout(T, H, I, k).total;
}

extern "C" moe_status moe_expert_ffn(const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                                     const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                                     const uint8_t* s_down, const float* g_scale, const float* topk_w,
                                     const int32_t* expert_count, const int32_t* expert_offset,
                                     const int32_t* active_experts, const int32_t* n_active,
                                     const int32_t* route_src, const int32_t* route_pos, int T, int H,
                                     int I, int E, int k, void* workspace, size_t workspace_bytes,
                                     uint16_t* y, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || E < 1 || k > E || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32 || H > 4096 || I > 4096) return MOE_ERR_UNSUPPORTED;
  const int chunks_h = H / 32, chunks_i = I / 32;
  const int lr_gu = lanes_per_row(chunks_h), lr_d = lanes_per_row(chunks_i);
  const int cpl_gu = chunks_h / lr_gu, cpl_d = chunks_i / lr_d;
  auto cpl_ok = [](int c) { return c == 1 || c == 2; };
  if (!cpl_ok(cpl_gu) || !cpl_ok(cpl_d)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                        expert_offset, active_experts, n_active, route_src, route_pos, workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  const WorkspaceLayout L = workspace_layout(T, H, I, k);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  FfnParams p;
  p.x = x; p.wg = w_gate; p.sg = s_gate; p.wu = w_up; p.su = s_up; p.wd = w_down; p.sd = s_down;
  p.gsc = g_scale; p.topk_w = topk_w; p.count = expert_count; p.offset = expert_offset;
  p.active = active_experts; p.n_active = n_active; p.route_src = route_src; p.route_pos = route_pos;
  p.T = T; p.H = H; p.I = I; p.E = E; p.k = k;
  p.h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.h_off);
  p.o = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.o_off);
  p.y = y;
  p.lr_gu = lr_gu;
  p.lr_d = lr_d;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int cus = device_cu_count();
  if (cus <= 0) return MOE_ERR_HIP;
  const long long max_active = std::min<long long>(E, (long long)T * k);
  const int rpt_gu = kWavesPerBlock * (kWave / lr_gu) * kU;
  const int rpt_d = kWavesPerBlock * (kWave / lr_d) * kU;
  const long long tasks_gu = max_active * ((I + rpt_gu - 1) / rpt_gu);
  const long long tasks_d = max_active * ((H + rpt_d - 1) / rpt_d);
  const int cap = cus * 4;
  const dim3 grid_gu((unsigned)std::min<long long>(tasks_gu, cap));
  const dim3 grid_d((unsigned)std::min<long long>(tasks_d, cap));

  if (cpl_gu == 1) gate_up_gemv<1, kU><<<grid_gu, kThreads, 0, s>>>(p);
  else gate_up_gemv<2, kU><<<grid_gu, kThreads, 0, s>>>(p);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  if (cpl_d == 1) down_gemv<1, kU><<<grid_d, kThreads, 0, s>>>(p);
  else down_gemv<2, kU><<<grid_d, kThreads, 0, s>>>(p);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const long long threads = (long long)T * (H / 2);
  combine_kernel<<<(unsigned)((threads + kThreads - 1) / kThreads), kThreads, 0, s>>>(p);
  return launch_status();
}
