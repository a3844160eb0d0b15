// Internal helpers shared by the HIP kernels and their host launchers.
// Written for gfx950 (CDNA4): 64-lane wavefronts, v_cvt_scalef32_pk_bf16_fp4,
// v_dot2_f32_bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- device

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32), and back (exact).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  return __builtin_bit_cast(bf16x2, u);
}

// Two FP4 E2M1 codes (byte B of `word`: low nibble = even element) -> two bf16
// in one instruction.  Scale 1.0: the conversion is exact (e2m1 values have
// at most 2 significant bits).
template <int B>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16x2(uint32_t word, float one = 1.0f) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, one, B);
}

// FP8 E4M3FN scale byte -> fp32 value * 2^-8, exactly.  Shifting the 7
// magnitude bits left by 7 gives the fp16 with the same fields (exponent bias
// 15 instead of 7, mantissa widened), i.e. value * 2^-8 for normals and
// subnormals alike; the fp16 -> fp32 conversion is exact.  The 2^8 is folded
// into the global scale.  Scale bytes are non-negative (sign bit clear) and
// never NaN (precondition).
__device__ __forceinline__ float e4m3_to_f32_div256(uint32_t byte) {
  const uint16_t h = (uint16_t)((byte & 0x7Fu) << 7);
  return (float)__builtin_bit_cast(_Float16, h);
}

// Fixed-order butterfly sum across the `width` lanes of an aligned lane group
// (width a power of two <= 64).  Every lane of the group ends with the sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// ---------------------------------------------------------------- host

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (cached per device id).
int device_cu_count();

inline moe_status launch_status() {
  hipError_t err = hipGetLastError();
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Largest power of two <= 64 dividing `chunks` (lanes that share one row).
inline int lanes_per_row(int chunks) {
  int l = 64;
  while (l > 1 && (chunks % l) != 0) l >>= 1;
  return l;
}

// Packed (MFMA tile order) weights: tiles of kPackRows rows, steps of kPackK
// along the reduction; per expert matrix the codes, then the scales, padded
// to 256 bytes.
constexpr int kPackRows = 128;
constexpr int kPackK = 64;
__host__ __device__ inline size_t packed_code_bytes(int N, int K) {
  return (size_t)((N + kPackRows - 1) / kPackRows) * kPackRows * (size_t)(K / 2);
}
__host__ __device__ inline size_t packed_matrix_bytes(int N, int K) {
  const size_t scales = (size_t)((N + kPackRows - 1) / kPackRows) * kPackRows * (size_t)(K / 16);
  return (packed_code_bytes(N, K) + scales + 255) & ~(size_t)255;
}

// Work lists of the expert kernels in the FFN workspace (see work_list.h).
struct WorkLists {
  int32_t* plan;      // MFMA items: [0] count, int4 items from [4]
  int32_t* rd_list;   // row-dot experts: [0] count, then the experts
  int plan_max;       // capacity of the MFMA item list
  int mfma_min;       // experts with at least this many routes take the MFMA kernels (0: none do)
  int rd_plan;        // the row-dot kernels read rd_list
  int32_t* queues;    // unit counters of the streaming down kernel (zeroed with the lists), or null
  int split_items;    // gate/up MFMA items take at most 64 routes when that makes at most this many items (0: never)
  int32_t* plan_down; // the down MFMA kernels' items, always chunks of up to 128 routes (layout of plan)
};

// A dense bf16 shared expert computed within a routed step (moe_step_shared):
// x [T,H], wg / wu [Is,H], wd [H,Is], h [T,Is] (workspace), y [T,H].  Its
// gate/up rows may ride along in the one-workgroup routing kernel and its
// down rows in the gate/up row-dot kernel, as extra workgroups of those
// launches.  gu_nc / dn_nc: 16-byte chunks per lane of a gate/up row
// (H / 512) and of a down row (Is / 512), 0 where that half cannot ride
// along (the ride-along code is compiled for gu_nc 1, 2, 4 and dn_nc 1, 2).
struct SharedRows {
  const uint16_t* x;
  const uint16_t* wg;
  const uint16_t* wu;
  const uint16_t* wd;
  uint16_t* h;
  uint16_t* y;
  int T, H, Is;
  int gu_nc, dn_nc;
};

// Argument checks of moe_shared_expert (no launch)
moe_status shared_check(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                        int T, int H, int Is, const void* workspace, size_t workspace_bytes, const uint16_t* y);
// The shared expert's own kernels: gate/up, then down
moe_status shared_gate_up(const SharedRows& s, hipStream_t st);
moe_status shared_down(const SharedRows& s, hipStream_t st);

// Whether moe_expert_ffn for these sizes reads work lists, and where they go
// in its workspace (*wl); *scratch_bytes = the workspace bytes in front of
// them, free until the expert kernels run.
bool ffn_work_lists(int T, int H, int I, int E, int k, bool packed, void* workspace, WorkLists* wl,
                    size_t* scratch_bytes);

// The expert FFN as in moe_expert_ffn_stage, with the packed weights (NULL:
// none; the MFMA tiles then read the standard layout).  lists_ready: the
// work lists were built by the bucketing (moe_step) for these buckets.  With
// `sr` (may be NULL; its gate/up rows already enqueued) the gate/up row-dot
// kernel also computes the shared expert's down rows; *sr_done says whether it
// did.
moe_status expert_ffn(int stage, const uint16_t* x, const uint8_t* w_gate, const uint8_t* s_gate,
                      const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const float* g_scale, const float* topk_w, const int32_t* expert_count,
                      const int32_t* expert_offset, const int32_t* active_experts, const int32_t* n_active,
                      const int32_t* route_src, const int32_t* route_pos, const uint8_t* packed, int T, int H,
                      int I, int E, int k, void* workspace, size_t workspace_bytes, uint16_t* y, hipStream_t s,
                      bool lists_ready = false, const SharedRows* sr = nullptr, bool* sr_done = nullptr);

// Routing and bucketing as in moe_route_bucket; `scratch` (may be NULL) is
// device memory the call may use until it returns (large batches bucket in
// parallel with it; moe_step lends the FFN workspace, unused at that point).
// With `wl` (may be NULL) the one-workgroup bucketing kernels also build the
// expert kernels' work lists; *lists_built says whether they did.  With `sr`
// (may be NULL) the one-workgroup routing kernel also computes the shared
// expert's gate/up rows; *sr_done says whether it did.
moe_status route_bucket(const float* logits, const float* bias, int T, int E, int k, int32_t* topk_idx,
                        float* topk_w, int32_t* expert_count, int32_t* expert_offset, int32_t* active_experts,
                        int32_t* n_active, int32_t* route_src, int32_t* route_pos, int32_t* scratch,
                        size_t scratch_bytes, hipStream_t s, const WorkLists* wl = nullptr,
                        bool* lists_built = nullptr, const SharedRows* sr = nullptr, bool* sr_done = nullptr);

// The small-batch step (moe_step up to 40 routes at H = 2048): the selection
// inside the gate/up launch (one workgroup per route and row tile, one more
// for the routing outputs), then the route-slot down/unroute.
// Outputs identical to route_bucket + expert_ffn.  Arguments already checked.
// stage 1: the selection and gate/up launch only; 2: the down/unroute launch
// only (after stage 1 on the same workspace); 3: both.  `side`: a shared
// expert whose rows ride along (small_step_side_ok), or null.
bool small_step_ok(int T, int H, int I, int E, int k);
// Whether a shared expert's rows can ride along in the small step's launches.
bool small_step_side_ok(int T, int H, int I, int E, int k, const SharedRows& sr);
moe_status small_step(const uint16_t* x, const float* logits, const float* bias, const uint8_t* w_gate,
                      const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                      const uint8_t* s_down, const float* g_scale, int T, int H, int I, int E, int k,
                      int32_t* topk_idx, float* topk_w, int32_t* expert_count, int32_t* expert_offset,
                      int32_t* active_experts, int32_t* n_active, int32_t* route_src, int32_t* route_pos,
                      void* workspace, uint16_t* y, hipStream_t s, int stage = 3,
                      const SharedRows* side = nullptr);

}  // namespace moe
