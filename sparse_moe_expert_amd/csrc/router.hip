// moe_router_logits: the router projection that produces the routing logits.
//
// logits[t, e] = fl32( sum_h x[t, h] * W_r[e, h] ).  The router is a
// projection followed by the selection (page "Persistent execution for
// Flash-Next GGUF on SM70", section "Router: selection and expert-task
// production"); its projection results span many workgroups, and the
// kernel boundary before moe_route_topk / moe_route_bucket is the hand-off
// to the selection.  Each bf16 x fp32 product is exact in fp64 (8 + 24
// significant bits), the sum is accumulated in fp64 and rounded once.
//
// Three kernels (gfx950): batches up to 64 tokens spread each expert row over
// one 256-lane workgroup (the router weights dominate the bytes); mid-size
// batches give each expert row one wavefront and chunks of 8 tokens; from
// 1024 tokens a register-tiled fp64 product (the arithmetic dominates).
#include "router_rows.h"

namespace moe {
namespace {

// Mid-size batches (64 < T < 1024): wavefront w of workgroup (b, c) owns
// expert row e = 4b + w and the workgroup's chunk of up to 8 tokens (rows
// staged in LDS); lane l holds the row's values h = 4(l + 64j) as fp64,
// converted once, forms a partial sum per token with v_fma_f64, and a
// fixed-order butterfly over the wavefront adds the 64 partials.
constexpr int kRtTokens = 8;           // tokens per workgroup of the chunked kernel

template <int NCH>
__global__ __launch_bounds__(kRtThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                   const float* __restrict__ w, int T, int H, int E,
                                                                   float* __restrict__ logits) {
  extern __shared__ __align__(16) uint16_t s_x[];   // [kRtTokens][H] bf16
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRtTokens;
  const int nt = min(kRtTokens, T - t0);
  const int e = blockIdx.x * kRtWaves + wave;
  const int nq = H / 4;                              // four-value pieces of a row
  // the wave's weight row (loads issued before the x staging completes)
  double wd[NCH][4];
  if (e < E) {
    const float4* wr = reinterpret_cast<const float4*>(w + (size_t)e * H);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = lane + kWave * j;
      const float4 v = q < nq ? wr[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      wd[j][0] = v.x; wd[j][1] = v.y; wd[j][2] = v.z; wd[j][3] = v.w;
    }
  }
  const int pieces = nt * (H / 8);                   // 16-byte pieces of the chunk's x rows
  const uint4* xs = reinterpret_cast<const uint4*>(x + (size_t)t0 * H);
  for (int i = threadIdx.x; i < pieces; i += kRtThreads) reinterpret_cast<uint4*>(s_x)[i] = xs[i];
  __syncthreads();
  if (e >= E) return;
  for (int t = 0; t < nt; ++t) {
    const uint16_t* xr = s_x + (size_t)t * H;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = lane + kWave * j;
      if (q < nq) {
        const uint2 b = *reinterpret_cast<const uint2*>(xr + 4 * q);
        acc = fma(wd[j][0], bf16_lo(b.x), acc);
        acc = fma(wd[j][1], bf16_hi(b.x), acc);
        acc = fma(wd[j][2], bf16_lo(b.y), acc);
        acc = fma(wd[j][3], bf16_hi(b.y), acc);
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) logits[(size_t)(t0 + t) * E + e] = (float)acc;
  }
}

// Large batches (T >= 1024): a register-tiled fp64 product.  A workgroup owns 64 tokens x
// 128 experts; thread (g, f) = (tid / 16, tid % 16) accumulates tokens
// 4g..4g+3 x experts 8f..8f+7 in 32 fp64 registers.  K advances 16 at a
// time: the chunk's activations and weights are converted to fp64 into LDS
// (k-major, so a thread's 4 tokens and 8 experts are contiguous), then each
// k adds 32 products per thread.  Each output is summed in k order.
constexpr int kRgTokens = 64, kRgExperts = 128, kRgK = 16;
constexpr int kRgMinTokens = 1024;     // from here the tiled product has enough workgroups

__global__ __launch_bounds__(kRtThreads) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ w, int T, int H, int E,
                                                                 float* __restrict__ logits) {
  __shared__ __align__(16) double s_x[kRgK][kRgTokens];
  __shared__ __align__(16) double s_w[kRgK][kRgExperts];
  const int tid = threadIdx.x;
  const int g = tid / 16, f = tid % 16;
  const int t0 = blockIdx.y * kRgTokens, e0 = blockIdx.x * kRgExperts;
  // staging roles: x piece (token tid/4, k 4*(tid%4)..+4), w piece (expert tid/2, k 8*(tid%2)..+8)
  const int xt = tid / 4, xk = 4 * (tid % 4);
  const int we = tid / 2, wk = 8 * (tid % 2);
  double acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  // global reads of one chunk (zeros past T, E or H; H is a multiple of 8)
  uint2 xb;
  float4 wa, wb;
  auto fetch = [&](int k0) {
    xb = make_uint2(0u, 0u);
    if (t0 + xt < T && k0 + xk < H) xb = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + xt) * H + k0 + xk);
    wa = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    wb = wa;
    if (e0 + we < E && k0 + wk < H) {
      wa = *reinterpret_cast<const float4*>(w + (size_t)(e0 + we) * H + k0 + wk);
      wb = *reinterpret_cast<const float4*>(w + (size_t)(e0 + we) * H + k0 + wk + 4);
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < H; k0 += kRgK) {
    __syncthreads();                                   // the previous chunk is consumed
    s_x[xk + 0][xt] = bf16_lo(xb.x);
    s_x[xk + 1][xt] = bf16_hi(xb.x);
    s_x[xk + 2][xt] = bf16_lo(xb.y);
    s_x[xk + 3][xt] = bf16_hi(xb.y);
    s_w[wk + 0][we] = wa.x; s_w[wk + 1][we] = wa.y; s_w[wk + 2][we] = wa.z; s_w[wk + 3][we] = wa.w;
    s_w[wk + 4][we] = wb.x; s_w[wk + 5][we] = wb.y; s_w[wk + 6][we] = wb.z; s_w[wk + 7][we] = wb.w;
    __syncthreads();
    if (k0 + kRgK < H) fetch(k0 + kRgK);               // in flight while this chunk is summed
#pragma unroll
    for (int k = 0; k < kRgK; ++k) {
      double a[4], b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = s_x[k][4 * g + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = s_w[k][8 * f + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + 8 * f + j;
      if (e < E) logits[(size_t)t * E + e] = (float)acc[i][j];
    }
  }
}

// tokens per pass: the smallest of 1, 2, 4, 8 that holds the batch (at most 8)
template <int NCH>
void launch_router_rows(int T, const uint16_t* x, const float* w, int H, int E, float* logits, hipStream_t s) {
  if (T <= 1) router_rows_kernel<NCH, 1><<<E, kRtThreads, 0, s>>>(x, w, T, H, E, logits);
  else if (T <= 2) router_rows_kernel<NCH, 2><<<E, kRtThreads, 0, s>>>(x, w, T, H, E, logits);
  else if (T <= 4) router_rows_kernel<NCH, 4><<<E, kRtThreads, 0, s>>>(x, w, T, H, E, logits);
  else router_rows_kernel<NCH, kRsGroup><<<E, kRtThreads, 0, s>>>(x, w, T, H, E, logits);
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E,
                                        float* logits, void* stream) {
  using namespace moe;
  if (T < 0 || E < 1 || H < 8 || H % 8 != 0) return MOE_ERR_INVALID_SHAPE;
  if (H > kRtMaxH || E > 1024) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits)) return MOE_ERR_MISALIGNED;
  if (((long long)T + kRgTokens - 1) / kRgTokens > 65535) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T <= kRsMaxTokens) {
    const int nc = (H / 8 + kRtThreads - 1) / kRtThreads;   // 16-byte pieces per thread
    if (nc <= 1) launch_router_rows<1>(T, x, w_router, H, E, logits, s);
    else launch_router_rows<2>(T, x, w_router, H, E, logits, s);
    return launch_status();
  }
  if (T >= kRgMinTokens) {
    const dim3 grid((unsigned)((E + kRgExperts - 1) / kRgExperts), (unsigned)((T + kRgTokens - 1) / kRgTokens));
    router_gemm_kernel<<<grid, kRtThreads, 0, s>>>(x, w_router, T, H, E, logits);
    return launch_status();
  }
  const dim3 grid((unsigned)((E + kRtWaves - 1) / kRtWaves), (unsigned)((T + kRtTokens - 1) / kRtTokens));
  const size_t dyn = (size_t)kRtTokens * H * 2;
  const int nch = (H / 4 + kWave - 1) / kWave;       // pieces per lane
  if (nch <= 1) router_logits_kernel<1><<<grid, kRtThreads, dyn, s>>>(x, w_router, T, H, E, logits);
  else if (nch <= 2) router_logits_kernel<2><<<grid, kRtThreads, dyn, s>>>(x, w_router, T, H, E, logits);
  else if (nch <= 4) router_logits_kernel<4><<<grid, kRtThreads, dyn, s>>>(x, w_router, T, H, E, logits);
  else if (nch <= 8) router_logits_kernel<8><<<grid, kRtThreads, dyn, s>>>(x, w_router, T, H, E, logits);
  else router_logits_kernel<16><<<grid, kRtThreads, dyn, s>>>(x, w_router, T, H, E, logits);
  return launch_status();
}
