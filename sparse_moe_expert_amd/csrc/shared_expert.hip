// Dense BF16 shared expert: y_t = W_down (SiLU(W_gate x_t) * (W_up x_t)) for
// every token (page "How I forked vLLM and made Qwen3.8-Flash-Next decode 1.6x
// faster on one GPU", section "2. FP8 for the dense layers": shared experts
// stay BF16; page "Persistent execution for Flash-Next GGUF on SM70", section
// "Opportunity sized from the actual routes": their work runs beside the
// routed experts').  Decode-sized batches make both projections matrix-vector
// products, bound by the weight bytes (3 * H * Is * 2).
//
// Two kernels, one wavefront per weight row (the row work is in
// shared_rows.h): gate/up writes h[t, r] = bf16(SiLU(W_gate[r] . x_t) *
// (W_up[r] . x_t)) to the workspace, down writes y[t, c] = bf16(W_down[c] .
// h_t).  Every sum has a fixed order: results are bitwise reproducible, and
// moe_step_shared, whose kernels run the same row work, gives the same bits.
#include "shared_rows.h"

namespace moe {
namespace {

constexpr int kSeThreads = 256;       // down: four waves, one weight row each
constexpr int kSeWaves = kSeThreads / kWave;
// gate/up: two waves (two rows of W_gate and W_up each) per workgroup, so
// that the rows' weight and activation reads spread over more compute units
constexpr int kSeGuThreads = 128;
constexpr int kSeGuWaves = kSeGuThreads / kWave;

template <int NC>
__global__ __launch_bounds__(kSeGuThreads) void shared_gate_up_kernel(SharedRows s) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * kSeGuWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= s.Is) return;
  se_gate_up_row<NC>(s, r, lane);
}

template <int NC>
__global__ __launch_bounds__(kSeThreads) void shared_down_kernel(SharedRows s) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = blockIdx.x * kSeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (c >= s.H) return;
  se_down_rows<NC, 1>(s, c, lane);
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

moe_status shared_gate_up(const SharedRows& sr, hipStream_t s) {
  const unsigned g = (unsigned)((sr.Is + kSeGuWaves - 1) / kSeGuWaves);
  switch (sr.H / 512) {
    case 1: shared_gate_up_kernel<1><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 2: shared_gate_up_kernel<2><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 3: shared_gate_up_kernel<3><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 4: shared_gate_up_kernel<4><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 5: shared_gate_up_kernel<5><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 6: shared_gate_up_kernel<6><<<g, kSeGuThreads, 0, s>>>(sr); break;
    case 7: shared_gate_up_kernel<7><<<g, kSeGuThreads, 0, s>>>(sr); break;
    default: shared_gate_up_kernel<8><<<g, kSeGuThreads, 0, s>>>(sr); break;
  }
  return launch_status();
}

moe_status shared_down(const SharedRows& sr, hipStream_t s) {
  const unsigned g = (unsigned)((sr.H + kSeWaves - 1) / kSeWaves);
  switch (sr.Is / 512) {
    case 1: shared_down_kernel<1><<<g, kSeThreads, 0, s>>>(sr); break;
    case 2: shared_down_kernel<2><<<g, kSeThreads, 0, s>>>(sr); break;
    case 3: shared_down_kernel<3><<<g, kSeThreads, 0, s>>>(sr); break;
    case 4: shared_down_kernel<4><<<g, kSeThreads, 0, s>>>(sr); break;
    case 5: shared_down_kernel<5><<<g, kSeThreads, 0, s>>>(sr); break;
    case 6: shared_down_kernel<6><<<g, kSeThreads, 0, s>>>(sr); break;
    case 7: shared_down_kernel<7><<<g, kSeThreads, 0, s>>>(sr); break;
    default: shared_down_kernel<8><<<g, kSeThreads, 0, s>>>(sr); break;
  }
  return launch_status();
}

moe_status shared_check(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                        int T, int H, int Is, const void* workspace, size_t workspace_bytes, const uint16_t* y) {
  if (T < 0 || H < 32 || Is < 32 || H % 32 != 0 || Is % 32 != 0) return MOE_ERR_INVALID_SHAPE;
  // one to eight 16-byte chunks per lane: rows of 512 .. 4096 values in steps of 512
  if (H % 512 != 0 || Is % 512 != 0 || H > 4096 || Is > 4096 || T > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, w_up, w_down, workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  if (workspace_bytes < align256((size_t)T * (size_t)Is * 2)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  // one buffer resource per tensor: byte counts must fit 31 bits
  if ((size_t)T * H * 2 >= 0x80000000ull || (size_t)T * Is * 2 >= 0x80000000ull ||
      (size_t)Is * H * 2 >= 0x80000000ull)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_shared_expert_workspace_size(int T, int H, int Is) {
  (void)H;
  if (T <= 0 || Is <= 0) return 0;
  return moe::align256((size_t)T * (size_t)Is * 2);
}

extern "C" moe_status moe_shared_expert(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                                        const uint16_t* w_down, int T, int H, int Is, void* workspace,
                                        size_t workspace_bytes, uint16_t* y, void* stream) {
  using namespace moe;
  const moe_status st = shared_check(x, w_gate, w_up, w_down, T, H, Is, workspace, workspace_bytes, y);
  if (st != MOE_OK || T == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const SharedRows sr{x, w_gate, w_up, w_down, static_cast<uint16_t*>(workspace), y, T, H, Is, 0, 0};
  if (shared_gate_up(sr, s) != MOE_OK) return MOE_ERR_HIP;
  return shared_down(sr, s);
}
