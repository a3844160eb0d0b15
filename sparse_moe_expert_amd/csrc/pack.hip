// moe_pack_weights: the expert weights rearranged offline into the order in
// which the MFMA tiles consume them, so that every weight load of those
// tiles is one contiguous kilobyte per wavefront.  The rearrangement of
// quantised bits to match the consumer's register fragments is the FLUTE
// technique (page "Persistent execution for Flash-Next GGUF on SM70",
// section "Primary sources and transferable mechanisms", paragraph "FLUTE").
// It is a pure byte permutation with zero padding; values are not touched.
//
// Layout of one matrix of one expert (N rows, reduction K): tiles of
// kPackRows = 128 rows, steps of kPackK = 64 along K, four wavefronts of 32
// rows per tile.  For tile t, step s, wave w and lane l (row r = 128t + 32w
// + l%32, half h = l/32):
//   codes  [t][s][w][l]  16 bytes: bytes 32s + 16h .. +16 of row r's codes
//   scales [t][s][w][l]   2 bytes: bytes 4s + 2h .. +2 of row r's scales
// (all codes of the matrix first, then all scales); rows r >= N are zeros.
// The packed buffer holds gate, up and down of every expert in that order:
// [gate e=0..E) [up e=0..E) [down e=0..E), each expert's matrix padded to
// 256 bytes.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;

// One thread per (tile, step, wave, lane) of one expert's matrix.
__global__ __launch_bounds__(kPackThreads) void pack_matrix_kernel(const uint8_t* __restrict__ codes,
                                                                   const uint8_t* __restrict__ scales, int E,
                                                                   int N, int K, uint8_t* __restrict__ out) {
  const int tiles = (N + kPackRows - 1) / kPackRows, steps = K / kPackK;
  const long long per_expert = (long long)tiles * steps * 4 * 64;         // slots of one expert
  const long long i = (long long)blockIdx.x * kPackThreads + threadIdx.x;
  if (i >= per_expert * E) return;
  const int e = (int)(i / per_expert);
  long long j = i - (long long)e * per_expert;
  const int l = (int)(j & 63);
  j >>= 6;
  const int w = (int)(j & 3);
  j >>= 2;
  const int s = (int)(j % steps), t = (int)(j / steps);
  const int r = t * kPackRows + w * 32 + (l & 31), h = l >> 5;
  const size_t code_row = (size_t)K / 2, scale_row = (size_t)K / 16;
  uint4 c = make_uint4(0u, 0u, 0u, 0u);
  uint16_t sc = 0;
  if (r < N) {
    c = *reinterpret_cast<const uint4*>(codes + ((size_t)e * N + r) * code_row + (size_t)s * 32 + (size_t)h * 16);
    sc = *reinterpret_cast<const uint16_t*>(scales + ((size_t)e * N + r) * scale_row + (size_t)s * 4 + (size_t)h * 2);
  }
  uint8_t* dst = out + (size_t)e * packed_matrix_bytes(N, K);
  reinterpret_cast<uint4*>(dst)[j * 256 + w * 64 + l] = c;
  reinterpret_cast<uint16_t*>(dst + packed_code_bytes(N, K))[j * 256 + w * 64 + l] = sc;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_packed_weights_size(int E, int H, int I) {
  if (E <= 0 || H <= 0 || I <= 0 || H % moe::kPackK != 0 || I % moe::kPackK != 0) return 0;
  return (size_t)E * (2 * moe::packed_matrix_bytes(I, H) + moe::packed_matrix_bytes(H, I));
}

extern "C" moe_status moe_pack_weights(const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                       const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down, int E,
                                       int H, int I, uint8_t* packed, void* stream) {
  using namespace moe;
  if (E < 1 || H < kPackK || I < kPackK || H % kPackK != 0 || I % kPackK != 0) return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || H > 4096 || I > 4096) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {w_gate, s_gate, w_up, s_up, w_down, s_down, packed};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_MISALIGNED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t gu = (size_t)E * packed_matrix_bytes(I, H);
  const struct {
    const uint8_t* c;
    const uint8_t* sc;
    int N, K;
    size_t at;
  } mats[3] = {{w_gate, s_gate, I, H, 0}, {w_up, s_up, I, H, gu}, {w_down, s_down, H, I, 2 * gu}};
  for (const auto& m : mats) {
    const long long slots = (long long)E * ((m.N + kPackRows - 1) / kPackRows) * (m.K / kPackK) * 4 * 64;
    const unsigned grid = (unsigned)((slots + kPackThreads - 1) / kPackThreads);
    pack_matrix_kernel<<<grid, kPackThreads, 0, s>>>(m.c, m.sc, E, m.N, m.K, packed + m.at);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  return MOE_OK;
}
