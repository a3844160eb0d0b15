// moe_step: one routed-MoE step (routing, bucketing, expert FFN with the
// weighted unroute) in one call.
//
// Small batches (at most 40 routes at H = 2048) take two kernels: the
// selection inside the gate/up launch (every workgroup, one per route and
// row tile, selects its token's experts itself; one more workgroup writes
// the routing outputs; no routing kernel, no hand-off), then the
// down/unroute with one slot per route.  Larger batches enqueue
// moe_route_bucket and then moe_expert_ffn on the caller's stream.  A one-kernel form of the step - every workgroup
// routing the batch itself, gate/up publishing each expert's intermediate
// through device-coherent stores and per-expert counters, down waiting on
// them, the last route of a token combining it - was built and measured on
// gfx950 and lost: the replicated routing is VALU-bound (all 1280
// workgroups select at once), and every cross-workgroup hand-off made while
// the weight stream is in flight waits behind that stream in the memory
// queues, so the hand-offs cost more than the kernel boundaries they remove.
// That pipeline is the one proposed for another machine on page "Persistent
// execution for Flash-Next GGUF on SM70" (section "First implementation
// boundary", steps 2-4; section "Primary sources and transferable
// mechanisms", paragraphs "MonoMoE" and "Hazy Research Megakernels", the
// latter noting that publication and readiness checks are a cost of their
// own).
#include <mutex>

#include "moe_common.h"

extern "C" size_t moe_step_workspace_size(int T, int H, int I, int E, int k) {
  return moe_expert_ffn_workspace_size(T, H, I, E, k);
}

// Host checks of the step with optional packed weights (NULL: none): every
// argument, before anything is launched.
static moe_status step_check(const uint16_t* x, const float* logits, const float* bias, const uint8_t* w_gate,
                             const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up,
                             const uint8_t* w_down, const uint8_t* s_down, const float* g_scale,
                             const uint8_t* packed, int T, int H, int I, int E, int k, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_count, int32_t* expert_offset,
                             int32_t* active_experts, int32_t* n_active, int32_t* route_src, int32_t* route_pos,
                             const void* workspace, size_t workspace_bytes, uint16_t* y) {
  // argument checks of the FFN call first, so that an invalid call launches nothing
  if (T < 0 || k < 1 || E < 1 || k > E || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return MOE_ERR_INVALID_SHAPE;
  if (E > 1024 || k > 32 || H > 4096 || I > 4096) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * H * 2 >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  // packed weights exist only for H and I multiples of the MFMA step
  if (packed && (H % moe::kPackK != 0 || I % moe::kPackK != 0)) return MOE_ERR_INVALID_SHAPE;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {x, logits, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_idx, topk_w,
                        expert_count, expert_offset, active_experts, n_active, route_src, route_pos,
                        workspace, y};
  for (const void* q : ptrs)
    if (!q) return MOE_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!moe::aligned16(q)) return MOE_ERR_MISALIGNED;
  if ((bias && !moe::aligned16(bias)) || (packed && !moe::aligned16(packed))) return MOE_ERR_MISALIGNED;
  if (workspace_bytes < moe_step_workspace_size(T, H, I, E, k)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

// The step with optional packed weights (NULL: none).
static moe_status step(const uint16_t* x, const float* logits, const float* bias, const uint8_t* w_gate,
                       const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                       const uint8_t* s_down, const float* g_scale, const uint8_t* packed, int T, int H, int I,
                       int E, int k, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                       int32_t* expert_offset, int32_t* active_experts, int32_t* n_active, int32_t* route_src,
                       int32_t* route_pos, void* workspace, size_t workspace_bytes, uint16_t* y, void* stream,
                       const moe::SharedRows* side = nullptr, int stage = 3) {
  const moe_status chk = step_check(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T,
                                    H, I, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts,
                                    n_active, route_src, route_pos, workspace, workspace_bytes, y);
  if (chk != MOE_OK || T == 0) return chk;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // small batches: the selection and the routing outputs inside the gate/up
  // launch (no routing kernel), then the route-slot down/unroute; a shared
  // expert's rows ride along in the same two launches where they fit
  if (side ? moe::small_step_side_ok(T, H, I, E, k, *side) : moe::small_step_ok(T, H, I, E, k))
    return moe::small_step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, T, H, I, E, k,
                           topk_idx, topk_w, expert_count, expert_offset, active_experts, n_active, route_src,
                           route_pos, workspace, y, s, stage, side);
  if (stage == 2)                                  // the expert FFN's second stage (it rebuilds its work lists)
    return moe::expert_ffn(2, x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                           expert_offset, active_experts, n_active, route_src, route_pos, packed, T, H, I, E, k,
                           workspace, workspace_bytes, y, s);
  // The expert kernels' work lists, when they read any, are built by the
  // one-workgroup bucketing kernel, which holds the counts already (one
  // launch less than building them in the FFN call).  The FFN workspace in
  // front of the lists is free until the expert kernels run: routing may use
  // it as scratch.
  moe::WorkLists wl;
  size_t scratch_bytes = workspace_bytes;
  const bool want_lists = moe::ffn_work_lists(T, H, I, E, k, packed != nullptr, workspace, &wl, &scratch_bytes);
  bool lists_built = false, gu_done = false, dn_done = false;
  moe_status st = moe::route_bucket(logits, bias, T, E, k, topk_idx, topk_w, expert_count, expert_offset,
                                    active_experts, n_active, route_src, route_pos, static_cast<int32_t*>(workspace),
                                    scratch_bytes, s, want_lists ? &wl : nullptr, &lists_built, side, &gu_done);
  if (st != MOE_OK) return st;
  // a shared expert's gate/up rows that did not ride along in the routing
  // kernel run on their own before the expert kernels (whose row-dot kernel
  // may carry its down rows)
  if (side && !gu_done && moe::shared_gate_up(*side, s) != MOE_OK) return MOE_ERR_HIP;
  st = moe::expert_ffn(stage, x, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, topk_w, expert_count,
                       expert_offset, active_experts, n_active, route_src, route_pos, packed, T, H, I, E, k,
                       workspace, workspace_bytes, y, s, lists_built, side, &dn_done);
  if (st != MOE_OK) return st;
  if (side && !dn_done) return moe::shared_down(*side, s);
  return MOE_OK;
}

extern "C" moe_status moe_step(const uint16_t* x, const float* logits, const float* bias,
                               const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                               const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                               const float* g_scale, int T, int H, int I, int E, int k,
                               int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                               int32_t* expert_offset, int32_t* active_experts, int32_t* n_active,
                               int32_t* route_src, int32_t* route_pos, void* workspace,
                               size_t workspace_bytes, uint16_t* y, void* stream) {
  return step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, nullptr, T, H, I, E, k, topk_idx,
              topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, workspace,
              workspace_bytes, y, stream);
}

extern "C" moe_status moe_step_packed(const uint16_t* x, const float* logits, const float* bias,
                                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                                      const float* g_scale, const uint8_t* packed, int T, int H, int I, int E,
                                      int k, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                                      int32_t* expert_offset, int32_t* active_experts, int32_t* n_active,
                                      int32_t* route_src, int32_t* route_pos, void* workspace,
                                      size_t workspace_bytes, uint16_t* y, void* stream) {
  if (!packed) return MOE_ERR_NULL_POINTER;
  return step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T, H, I, E, k, topk_idx,
              topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, workspace,
              workspace_bytes, y, stream);
}

// The step and a dense bf16 shared expert of the same tokens: y as
// moe_step(_packed) computes it, y_shared as moe_shared_expert does, bit for
// bit.  At decode sizes the shared expert's rows ride along in the step's own
// launches instead of two kernels of their own: in the small step (up to 40
// routes at H = 2048) gate/up in the selection launch and down in the
// route-slot down/unroute; otherwise gate/up in the routing kernel and down
// in the gate/up row-dot kernel.
extern "C" moe_status moe_step_shared(const uint16_t* x, const float* logits, const float* bias,
                                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                                      const float* g_scale, const uint8_t* packed, int T, int H, int I, int E,
                                      int k, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                                      int32_t* expert_offset, int32_t* active_experts, int32_t* n_active,
                                      int32_t* route_src, int32_t* route_pos, void* workspace,
                                      size_t workspace_bytes, uint16_t* y, const uint16_t* se_gate,
                                      const uint16_t* se_up, const uint16_t* se_down, int Is, void* se_workspace,
                                      size_t se_workspace_bytes, uint16_t* y_shared, void* stream) {
  const moe_status st = moe::shared_check(x, se_gate, se_up, se_down, T, H, Is, se_workspace, se_workspace_bytes,
                                          y_shared);
  if (st != MOE_OK) return st;
  const int gu = H / 512, dn = Is / 512;
  const moe::SharedRows side{x, se_gate, se_up, se_down, static_cast<uint16_t*>(se_workspace), y_shared, T, H, Is,
                             (gu == 1 || gu == 2 || gu == 4) ? gu : 0, (dn == 1 || dn == 2) ? dn : 0};
  return step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T, H, I, E, k, topk_idx,
              topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, workspace,
              workspace_bytes, y, stream, &side);
}

// ------------------------------------------------------------------ no allocation

// The workspace of moe_step_noalloc: a static device array, one copy per GPU
// the library runs on, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels receive the address
// that hipGetSymbolAddress returns for the current device (scratch_on_device).
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first
// call on each device (with that device current) and kept.
moe_status scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_step_noalloc(const uint16_t* x, const float* logits, const float* bias,
                                       const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                       const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                                       const float* g_scale, const uint8_t* packed, int T, int H, int I, int E,
                                       int k, int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                                       int32_t* expert_offset, int32_t* active_experts, int32_t* n_active,
                                       int32_t* route_src, int32_t* route_pos, uint16_t* y, void* stream) {
  // every host check first, against the scratch size (a stand-in aligned
  // address: nothing is dereferenced on the host)
  const void* stand_in = reinterpret_cast<const void*>(uintptr_t(256));
  const moe_status chk = step_check(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T,
                                    H, I, E, k, topk_idx, topk_w, expert_count, expert_offset, active_experts,
                                    n_active, route_src, route_pos, stand_in, kNoAllocScratchBytes, y);
  if (chk == MOE_ERR_WORKSPACE_TOO_SMALL) return MOE_ERR_SCRATCH_TOO_SMALL;
  if (chk != MOE_OK || T == 0) return chk;
  void* ws = nullptr;
  const moe_status st = scratch_on_device(&ws);
  if (st != MOE_OK) return st;
  return step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T, H, I, E, k, topk_idx,
              topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, ws,
              kNoAllocScratchBytes, y, stream);
}

extern "C" moe_status moe_step_stage(int stage, const uint16_t* x, const float* logits, const float* bias,
                                     const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                     const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                                     const float* g_scale, const uint8_t* packed, int T, int H, int I, int E, int k,
                                     int32_t* topk_idx, float* topk_w, int32_t* expert_count,
                                     int32_t* expert_offset, int32_t* active_experts, int32_t* n_active,
                                     int32_t* route_src, int32_t* route_pos, void* workspace,
                                     size_t workspace_bytes, uint16_t* y, void* stream) {
  if (stage < 1 || stage > 3) return MOE_ERR_INVALID_SHAPE;
  return step(x, logits, bias, w_gate, s_gate, w_up, s_up, w_down, s_down, g_scale, packed, T, H, I, E, k, topk_idx,
              topk_w, expert_count, expert_offset, active_experts, n_active, route_src, route_pos, workspace,
              workspace_bytes, y, stream, nullptr, stage);
}
