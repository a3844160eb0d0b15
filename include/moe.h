/*
 * Routed NVFP4 mixture-of-experts FFN for one MI355X (gfx950): C ABI.
 *
 * One routed-MoE step of a decode/verify/prefill batch is three calls on one
 * stream:
 *   moe_route_topk     router logits -> top-k expert ids and gate weights
 *   moe_bucket_routes  top-k ids -> routes grouped by expert (stable order)
 *   moe_expert_ffn     bf16 tokens + NVFP4 experts + buckets -> bf16 output
 * or the same step in one call, moe_step (two kernels for small batches).
 * The router projection that produces the logits is a prerequisite outside
 * these calls (the MonoMoE host wrapper takes precomputed router logits and
 * the SM70 design note keeps the router GEMV as an explicit prerequisite:
 * page "Persistent execution for Flash-Next GGUF on SM70", sections "MonoMoE"
 * and "First implementation boundary"); moe_router_logits computes it on the
 * GPU for callers that start from the tokens.
 *
 * Conventions for every call
 *  - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous, aligned to 16 bytes (MOE_ERR_MISALIGNED otherwise).  Scalars
 *    (sizes) are passed by value.
 *  - A call only enqueues kernels on `stream` (a hipStream_t passed as void*;
 *    NULL = the null stream).  No call allocates, frees, synchronises, prints
 *    or keeps per-call host state, so the three calls can be captured into a
 *    HIP graph and replayed with new input contents.
 *  - Arguments are checked on the host before any launch; on error nothing is
 *    launched and a status other than MOE_OK is returned.  Device-side faults
 *    surface as HIP errors at the caller's next synchronisation.
 *  - Preconditions the host cannot check (device data): logits and activations
 *    are finite; topk_idx values lie in [0, E); bucket arrays are the output
 *    of moe_bucket_routes for the same topk_idx.
 *  - Results are bitwise reproducible for identical inputs: no floating-point
 *    atomics; every reduction has a fixed order.
 *  - Calls are reentrant.  Concurrent calls need distinct outputs and
 *    workspaces.
 */
#ifndef SPARSE_MOE_EXPERT_AMD_MOE_H
#define SPARSE_MOE_EXPERT_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  MOE_ERR_INVALID_SHAPE = 2,       /* T < 0, k < 1, k > E, H or I not a multiple of 32 ... */
  MOE_ERR_UNSUPPORTED = 3,         /* outside the supported envelope (see each call) */
  MOE_ERR_MISALIGNED = 4,          /* a tensor pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < moe_expert_ffn_workspace_size() */
  MOE_ERR_HIP = 6,                 /* a HIP runtime call failed (launch or device query) */
  MOE_ERR_SCRATCH_TOO_SMALL = 7    /* moe_step_noalloc: the sizes need more than its static scratch */
} moe_status;

/*
 * moe_router_logits — the router projection: tokens -> routing logits.
 *
 * Defines logits[t,e] = fl32( sum_h x[t,h] * w_router[e,h] ): every bf16
 * activation and fp32 weight is exact in fp64, so is each product; the sum
 * is accumulated in fp64 and rounded once to fp32.  The router is this
 * projection followed by the selection of moe_route_topk (page "Persistent
 * execution for Flash-Next GGUF on SM70", section "Router: selection and
 * expert-task production", which also notes that the projection's results
 * span many workgroups and need an explicit hand-off to the selection: here
 * the boundary between this call and the next on the stream).  The fp64 sum
 * is taken in a fixed order, so results are bitwise reproducible; against
 * the exactly rounded value a logit can differ by one fp32 ulp, when the
 * exact sum lies within the fp64 accumulation error of a rounding boundary.
 *
 *   x         [T, H] bf16 bits     in
 *   w_router  [E, H] fp32          in
 *   logits    [T, E] fp32          out
 * Shapes: T >= 0 (T = 0 launches nothing), E >= 1, H >= 8 and a multiple of
 * 8 (else MOE_ERR_INVALID_SHAPE).  Envelope: H <= 4096, E <= 1024,
 * T <= 4194240 (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_router_logits(const uint16_t* x, const float* w_router,
                             int T, int H, int E, float* logits,
                             void* stream);

/*
 * moe_route_topk — softmax top-k routing with renormalised gate weights.
 *
 * Defines: per token the experts are scored z[t,e] = fl32(logits[t,e] +
 * bias[e]) (one fp32 add; z = logits when bias is NULL).  The k largest z are
 * chosen by repeated arg-max; equal scores go to the lower expert id, and
 * -0.0 equals +0.0 (page "How I forked vLLM and made Qwen3.8-Flash-Next
 * decode 1.6x faster on one GPU", section "5. Hand-written kernels",
 * paragraph "Fused MoE routing"; page "Persistent execution for Flash-Next
 * GGUF on SM70", section "Router: selection and expert-task production").
 * Slot j holds the j-th choice (z descending, id ascending).  Gate weights
 * are the softmax over all E experts renormalised over the chosen k, i.e.
 * topk_w[t,j] = exp(z_j - z_0) / sum_i exp(z_i - z_0) over the chosen i,
 * computed in fp32 (|error| <= 1e-6 against exact arithmetic).
 *
 *   logits    [T, E] fp32          in
 *   bias      [E] fp32 or NULL     in
 *   topk_idx  [T, k] int32         out
 *   topk_w    [T, k] fp32          out, each row sums to 1 (to rounding)
 * Shapes: T >= 0 (T = 0 launches nothing), 1 <= k <= E.  Envelope:
 * E <= 1024, k <= 32 (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_route_topk(const float* logits, const float* bias,
                          int T, int E, int k,
                          int32_t* topk_idx, float* topk_w,
                          void* stream);

/*
 * moe_bucket_routes — group the R = T*k routes by expert.
 *
 * Defines the counts, scan, expert ids and scatter that follow top-k in the
 * fused routing kernel (page "How I forked vLLM and made Qwen3.8-Flash-Next
 * decode 1.6x faster on one GPU", section "5. Hand-written kernels",
 * paragraph "Fused MoE routing") as the compact expert-presence list and
 * original route positions asked for by the SM70 design note (page
 * "Persistent execution for Flash-Next GGUF on SM70", section "First
 * implementation boundary", step 1).  A route is named by its flat id
 * r = t*k + j.  Integer-only and exact:
 *   expert_count   [E]    out  routes per expert
 *   expert_offset  [E+1]  out  exclusive prefix sum of expert_count
 *   active_experts [E]    out  ascending ids with count > 0, then -1
 *   n_active       [1]    out  number of ids with count > 0
 *   route_src      [R]    out  flat route ids ordered by (expert, r)
 *   route_pos      [R]    out  inverse: route_pos[route_src[p]] == p
 * Shapes: T >= 0 (T = 0 launches nothing), 1 <= k <= E.  Envelope:
 * E <= 1024, R <= 2^24 (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_bucket_routes(const int32_t* topk_idx, int T, int E, int k,
                             int32_t* expert_count, int32_t* expert_offset,
                             int32_t* active_experts, int32_t* n_active,
                             int32_t* route_src, int32_t* route_pos,
                             void* stream);

/*
 * moe_route_bucket — moe_route_topk followed by moe_bucket_routes, fused.
 *
 * Same arguments, outputs, envelope and errors as the two calls in sequence
 * (outputs are identical bit for bit).  For T <= 16 with T*k <= 256 and
 * E <= 512 both steps run in one workgroup of one kernel, the fused routing
 * kernel's design for small batches (page "How I forked vLLM and made
 * Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section "5. Hand-written
 * kernels", paragraph "Fused MoE routing"); larger batches run the selection
 * over the chip, then the bucketing: one workgroup up to 1024 routes, one
 * launch of one workgroup per 1024-route chunk up to 65536.
 */
moe_status moe_route_bucket(const float* logits, const float* bias,
                            int T, int E, int k,
                            int32_t* topk_idx, float* topk_w,
                            int32_t* expert_count, int32_t* expert_offset,
                            int32_t* active_experts, int32_t* n_active,
                            int32_t* route_src, int32_t* route_pos,
                            void* stream);

/*
 * moe_router_route_bucket — moe_router_logits, moe_route_topk and
 * moe_bucket_routes in one call: tokens -> logits -> top-k ids and gate
 * weights -> route buckets, outputs identical bit for bit to the three calls
 * in sequence.  Small batches (T <= 16, T*k <= 256, E <= 512) run all of it in one
 * launch: the router's projection spans many workgroups, so the fused kernel
 * hands its results to the selection explicitly (page "Persistent execution
 * for Flash-Next GGUF on SM70", section "Router: selection and expert-task
 * production"): each workgroup makes its logits visible at device scope and
 * counts itself in `counter`; the last one to arrive routes and buckets the
 * batch and sets `counter` back to 0.  No workgroup waits for another.
 * Larger batches run the projection and moe_route_bucket back to back.
 * Measured on one MI355X at T = 4, H = 2048, E = 512, k = 10: the one-launch
 * form takes ~11.7 us against 4.7 + 4.3 us for the projection and routing
 * kernels it replaces (the device-scope hand-off - an L2 write-back and
 * invalidate around one atomic per workgroup - costs more than the kernel
 * boundary); for latency prefer moe_router_logits then moe_step.
 *   x, w_router, logits        as for moe_router_logits (logits is an output)
 *   bias, k, topk_idx, topk_w  as for moe_route_topk
 *   expert_count ... route_pos as for moe_bucket_routes
 *   counter   [1] int32, device memory owned by the caller: 0 before the
 *             first call (e.g. allocated zeroed); every call leaves it 0, so
 *             the call can be captured in a graph and replayed.  Concurrent
 *             calls need distinct counters.
 * Shapes and envelope: those of the three calls (H a multiple of 8 up to
 * 4096, E <= 1024, k <= 32, R <= 2^24); every check runs before any launch.
 */
moe_status moe_router_route_bucket(const uint16_t* x, const float* w_router, const float* bias,
                                   int T, int H, int E, int k, float* logits,
                                   int32_t* topk_idx, float* topk_w,
                                   int32_t* expert_count, int32_t* expert_offset,
                                   int32_t* active_experts, int32_t* n_active,
                                   int32_t* route_src, int32_t* route_pos,
                                   int32_t* counter, void* stream);

/*
 * Bytes of device workspace moe_expert_ffn needs for these sizes (0 when
 * T == 0 or a size is not positive): the per-route intermediates, 2*I + 2*H
 * bytes per route; the dense kernels' two work lists (gate/up and down),
 * each 16 bytes for each of at most min(E, T*k) + T*k/128 items (rounded up
 * to a multiple of 8) plus 16;
 * the row-dot kernels' expert list, 4 bytes for each of min(E, T*k)
 * experts plus 4; and the streaming down kernel's unit counters, 9 of them
 * 128 bytes apart (1152 bytes); each region rounded up to 256 bytes.
 */
size_t moe_expert_ffn_workspace_size(int T, int H, int I, int E, int k);

/*
 * moe_expert_ffn — routed NVFP4 SwiGLU experts with a weighted unroute.
 *
 * Defines, per route p = (t, j) with expert e = topk_idx[t,j] (page
 * "Persistent execution for Flash-Next GGUF on SM70", sections "What the
 * measurements establish" and "First implementation boundary"):
 *   h_p = SiLU(Wg_e x_t) * (Wu_e x_t),   o_p = Wd_e h_p,
 *   y_t = sum_{j=0}^{k-1} topk_w[t,j] * o_(t,j), summed in slot order j
 *         (a fixed order, never arrival order), rounded once to bf16 (RNE).
 * Each active expert's weights are streamed from HBM once per call for all
 * of its routes (unique-expert reuse).  Accumulation is fp32; h is kept as
 * bf16 between the two projections; where a route's down output o_p goes
 * through memory (batches too large for the fused small-batch kernel) it is
 * rounded once to fp16 before the fp32 weighting (the per-route FP16 down
 * rounding of the SM70 design note, step 4).
 *
 * NVFP4 weights: element = e2m1 * e4m3 * global.  e2m1 codes are packed two
 * per byte, element 2i in the low nibble of byte i; one e4m3 (OCP E4M3FN)
 * scale per 16 consecutive elements along the reduction dimension; one fp32
 * global scale per matrix.
 *   x           [T, H] bf16 bits        in
 *   w_gate/w_up [E, I, H/2] uint8       in   (rows = outputs, along H)
 *   s_gate/s_up [E, I, H/16] uint8      in
 *   w_down      [E, H, I/2] uint8       in   (rows = outputs, along I)
 *   s_down      [E, H, I/16] uint8      in
 *   g_scale     [E, 3] fp32             in   (gate, up, down global scales)
 *   topk_w      [T, k] fp32             in   (from moe_route_topk)
 *   expert_count, expert_offset, active_experts, n_active, route_src,
 *   route_pos                           in   (from moe_bucket_routes)
 *   workspace   device buffer of workspace_bytes >= moe_expert_ffn_workspace_size(T,H,I,E,k),
 *               owned by the caller; holds the per-route intermediates h
 *               (bf16 [T*k, I]) and o (fp16 [T*k, H]) and the work lists
 *               of the expert kernels.  Its contents before and after a
 *               call are unspecified and never need a reset.
 *   y           [T, H] bf16 bits        out
 * Shapes: T >= 0 (T = 0 launches nothing), 1 <= k <= E, H and I multiples of
 * 32.  Envelope: E <= 1024, k <= 32, H and I from 32 to 4096 (H/32 and I/32
 * need not be powers of two: the Flash-Next expert, H = 2560 and I = 640,
 * qualifies), T*H*2 < 2^31 (the activations are addressed with 32-bit
 * offsets); else MOE_ERR_UNSUPPORTED.
 */
moe_status moe_expert_ffn(const uint16_t* x,
                          const uint8_t* w_gate, const uint8_t* s_gate,
                          const uint8_t* w_up, const uint8_t* s_up,
                          const uint8_t* w_down, const uint8_t* s_down,
                          const float* g_scale,
                          const float* topk_w,
                          const int32_t* expert_count, const int32_t* expert_offset,
                          const int32_t* active_experts, const int32_t* n_active,
                          const int32_t* route_src, const int32_t* route_pos,
                          int T, int H, int I, int E, int k,
                          void* workspace, size_t workspace_bytes,
                          uint16_t* y,
                          void* stream);

/*
 * moe_expert_ffn_stage — one stage of moe_expert_ffn, same arguments.
 *   stage 1: gate/up + SiLU * multiply only; leaves h in the workspace.
 *   stage 2: down + weighted unroute only; reads h from the workspace, which
 *            must hold stage 1's result for the same routes and inputs.
 *   stage 3: both (exactly moe_expert_ffn).
 * Any other stage returns MOE_ERR_INVALID_SHAPE.  Lets a caller time or
 * interleave the two streaming phases separately.
 */
moe_status moe_expert_ffn_stage(int stage,
                                const uint16_t* x,
                                const uint8_t* w_gate, const uint8_t* s_gate,
                                const uint8_t* w_up, const uint8_t* s_up,
                                const uint8_t* w_down, const uint8_t* s_down,
                                const float* g_scale,
                                const float* topk_w,
                                const int32_t* expert_count, const int32_t* expert_offset,
                                const int32_t* active_experts, const int32_t* n_active,
                                const int32_t* route_src, const int32_t* route_pos,
                                int T, int H, int I, int E, int k,
                                void* workspace, size_t workspace_bytes,
                                uint16_t* y,
                                void* stream);

/*
 * Bytes of device workspace moe_step needs for these sizes (0 when T == 0);
 * equal to moe_expert_ffn_workspace_size.
 */
size_t moe_step_workspace_size(int T, int H, int I, int E, int k);

/*
 * moe_step — one whole routed-MoE step: moe_route_topk, moe_bucket_routes
 * and moe_expert_ffn in one call, with the same inputs and outputs (all
 * identical to what those calls produce).  It enqueues moe_route_bucket and
 * then moe_expert_ffn on `stream`.
 *   x, w_*, s_*, g_scale  in   as for moe_expert_ffn
 *   logits, bias          in   as for moe_route_topk
 *   topk_idx, topk_w      out  as from moe_route_topk
 *   expert_count ... route_pos  out  as from moe_bucket_routes
 *   workspace             >= moe_step_workspace_size(T,H,I,E,k) bytes, owned
 *                         by the caller, as for moe_expert_ffn
 *   y                     [T, H] bf16 bits out
 * Shapes, envelope and errors: those of the three calls; arguments are all
 * checked before anything is launched.
 */
moe_status moe_step(const uint16_t* x, const float* logits, const float* bias,
                    const uint8_t* w_gate, const uint8_t* s_gate,
                    const uint8_t* w_up, const uint8_t* s_up,
                    const uint8_t* w_down, const uint8_t* s_down,
                    const float* g_scale,
                    int T, int H, int I, int E, int k,
                    int32_t* topk_idx, float* topk_w,
                    int32_t* expert_count, int32_t* expert_offset,
                    int32_t* active_experts, int32_t* n_active,
                    int32_t* route_src, int32_t* route_pos,
                    void* workspace, size_t workspace_bytes,
                    uint16_t* y,
                    void* stream);

/*
 * moe_step_stage — one part of moe_step / moe_step_packed (`packed` may be
 * NULL), same arguments, so that a caller can time the step's phases:
 *   stage 1: everything up to and including the gate/up projection (for
 *            small batches the launch that selects and computes gate/up; for
 *            larger ones the routing and bucketing kernels and the gate/up
 *            kernels);
 *   stage 2: the rest (down projection and weighted unroute); reads what
 *            stage 1 left in the outputs and the workspace for the same
 *            inputs;
 *   stage 3: the whole step (exactly moe_step / moe_step_packed).
 * Stages 1 then 2 give moe_step's outputs bit for bit.  Any other stage
 * returns MOE_ERR_INVALID_SHAPE; every other check as for moe_step.
 */
moe_status moe_step_stage(int stage, const uint16_t* x, const float* logits, const float* bias,
                          const uint8_t* w_gate, const uint8_t* s_gate,
                          const uint8_t* w_up, const uint8_t* s_up,
                          const uint8_t* w_down, const uint8_t* s_down,
                          const float* g_scale, const uint8_t* packed,
                          int T, int H, int I, int E, int k,
                          int32_t* topk_idx, float* topk_w,
                          int32_t* expert_count, int32_t* expert_offset,
                          int32_t* active_experts, int32_t* n_active,
                          int32_t* route_src, int32_t* route_pos,
                          void* workspace, size_t workspace_bytes,
                          uint16_t* y, void* stream);

/*
 * Bytes of the packed copy of all expert weights that moe_pack_weights
 * writes for these sizes (0 when H or I is not a multiple of 64, or a size
 * is not positive).
 */
size_t moe_packed_weights_size(int E, int H, int I);

/*
 * moe_pack_weights — the expert weights rearranged into the order in which
 * the MFMA tiles of moe_step_packed read them (quantised bits rearranged
 * offline to match the consumer's register fragments, as FLUTE does: page
 * "Persistent execution for Flash-Next GGUF on SM70", section "Primary
 * sources and transferable mechanisms", paragraph "FLUTE").  A pure byte
 * permutation with zero padding: every code and scale byte is copied
 * unchanged.  Done once when the weights are loaded; the packed copy is
 * read instead of the standard layout by the MFMA tiles (experts with many
 * routes), which then load one contiguous kilobyte per wavefront.
 *   w_*, s_*   in   standard layout, as for moe_expert_ffn
 *   packed     out  device buffer of moe_packed_weights_size(E,H,I) bytes,
 *                   owned by the caller.  Layout per matrix and expert (N
 *                   rows, reduction K; gate and up: N = I, K = H; down:
 *                   N = H, K = I): 128-row tiles t, 64-wide reduction steps
 *                   s, four 32-row groups w, 64 lanes l (row 128t + 32w +
 *                   l%32, half h = l/32): 16 code bytes 32s+16h.. of the row
 *                   at index ((t*S + s)*4 + w)*64 + l, then all scales (2
 *                   bytes 4s+2h.. at the same index); rows past N are zero;
 *                   each expert's matrix padded to 256 bytes; gate of all
 *                   experts, then up, then down.
 * Shapes: H and I multiples of 64 (else MOE_ERR_INVALID_SHAPE); envelope
 * as for moe_expert_ffn.
 */
moe_status moe_pack_weights(const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up,
                            const uint8_t* w_down, const uint8_t* s_down,
                            int E, int H, int I, uint8_t* packed, void* stream);

/*
 * moe_step_packed — moe_step with the packed copy of the same weights
 * (from moe_pack_weights; must not be NULL).  Results are identical to
 * moe_step's; only the MFMA tiles' weight loads change.  H and I must be
 * multiples of 64.
 */
moe_status moe_step_packed(const uint16_t* x, const float* logits, const float* bias,
                           const uint8_t* w_gate, const uint8_t* s_gate,
                           const uint8_t* w_up, const uint8_t* s_up,
                           const uint8_t* w_down, const uint8_t* s_down,
                           const float* g_scale, const uint8_t* packed,
                           int T, int H, int I, int E, int k,
                           int32_t* topk_idx, float* topk_w,
                           int32_t* expert_count, int32_t* expert_offset,
                           int32_t* active_experts, int32_t* n_active,
                           int32_t* route_src, int32_t* route_pos,
                           void* workspace, size_t workspace_bytes,
                           uint16_t* y,
                           void* stream);

/*
 * Bytes of device workspace moe_shared_expert needs (0 when T <= 0): the
 * intermediate h, T*Is bf16 values, rounded up to 256 bytes.
 */
size_t moe_shared_expert_workspace_size(int T, int H, int Is);

/*
 * moe_shared_expert — the dense shared expert that every token goes through,
 * beside the routed ones, with BF16 weights (page "How I forked vLLM and made
 * Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section "2. FP8 for the
 * dense layers"; page "Persistent execution for Flash-Next GGUF on SM70",
 * section "Opportunity sized from the actual routes", on running it beside
 * the routed work):
 *   h_t = bf16(SiLU(W_gate x_t) * (W_up x_t)),   y_t = bf16(W_down h_t)
 * with fp32 accumulation, sums in a fixed order (bitwise reproducible).  The
 * caller adds y to the routed output; to overlap the two, enqueue this call
 * on a second stream.
 *   x          [T, H] bf16 bits         in
 *   w_gate     [Is, H] bf16 bits        in   (rows = outputs)
 *   w_up       [Is, H] bf16 bits        in
 *   w_down     [H, Is] bf16 bits        in
 *   workspace  >= moe_shared_expert_workspace_size(T, H, Is) bytes, owned by
 *              the caller, contents unspecified before and after
 *   y          [T, H] bf16 bits         out
 * Shapes: T >= 0 (T = 0 launches nothing), H and Is multiples of 32 (else
 * MOE_ERR_INVALID_SHAPE).  Envelope: H and Is multiples of 512 up to 4096,
 * T <= 2^20 (else MOE_ERR_UNSUPPORTED).  Decode-sized batches: the tokens
 * are taken four at a time by every weight row.
 */
moe_status moe_shared_expert(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                             const uint16_t* w_down, int T, int H, int Is,
                             void* workspace, size_t workspace_bytes,
                             uint16_t* y, void* stream);

/*
 * moe_step_shared — one routed step and the dense shared expert of the same
 * tokens in one call (page "Persistent execution for Flash-Next GGUF on
 * SM70", section "Opportunity sized from the actual routes": the shared
 * expert's work runs beside the routed experts'; page "How I forked vLLM and
 * made Qwen3.8-Flash-Next decode 1.6x faster on one GPU", section "2. FP8
 * for the dense layers": its weights stay BF16).
 *   Arguments up to y: as moe_step, plus `packed` (NULL: none) as in
 *              moe_step_packed.  y receives the routed output, bit for bit
 *              what moe_step / moe_step_packed writes.
 *   se_gate, se_up [Is, H], se_down [H, Is], se_workspace, y_shared: as
 *              w_gate, w_up, w_down, workspace and y of moe_shared_expert;
 *              y_shared receives bit for bit what moe_shared_expert writes.
 *              The caller adds y and y_shared.  No output may overlap
 *              another output or an input.
 * The shared expert's argument checks come first, then the step's; a
 * failing check launches nothing.  Where the step takes its two-launch form
 * (at most 40 routes at H = 2048, rows of I of one 16-byte chunk per lane),
 * Is is 512 or 1024 and T * Is * 2 bytes fit the down launch's LDS, the
 * shared gate/up rows run as extra workgroups of the selection launch and
 * its down rows in the last waves of the down/unroute workgroups.  Other
 * decode sizes (at most 16 tokens and 256 routes with at most 512 experts;
 * H of 512, 1024 or 2048 for the gate/up rows, Is of 512 or 1024 for the
 * down rows) run the shared rows as extra workgroups of the step's routing
 * and gate/up launches; otherwise its own two kernels run on the same
 * stream.
 */
moe_status moe_step_shared(const uint16_t* x, const float* logits, const float* bias,
                           const uint8_t* w_gate, const uint8_t* s_gate,
                           const uint8_t* w_up, const uint8_t* s_up,
                           const uint8_t* w_down, const uint8_t* s_down,
                           const float* g_scale, const uint8_t* packed,
                           int T, int H, int I, int E, int k,
                           int32_t* topk_idx, float* topk_w,
                           int32_t* expert_count, int32_t* expert_offset,
                           int32_t* active_experts, int32_t* n_active,
                           int32_t* route_src, int32_t* route_pos,
                           void* workspace, size_t workspace_bytes, uint16_t* y,
                           const uint16_t* se_gate, const uint16_t* se_up,
                           const uint16_t* se_down, int Is,
                           void* se_workspace, size_t se_workspace_bytes,
                           uint16_t* y_shared, void* stream);

/*
 * moe_expert_ffn_per_route — the routed experts without unique-expert reuse:
 * the baseline of the reuse measurement on page "Persistent execution for
 * Flash-Next GGUF on SM70" (section "Measurements that can accept or reject
 * the design": variants on the same storage and decoder; section
 * "Opportunity sized from the actual routes": bytes issued per route against
 * the distinct experts' bytes).  Every route (t, j) streams the weights of
 * its expert topk_idx[t, j] itself (an expert picked by n tokens is read n
 * times); no bucket arrays are used.  Same result definition as
 * moe_expert_ffn (h in bf16, each route's down output rounded once to fp16,
 * y summed in slot order in fp32 and rounded once to bf16).
 *   x, w_*, s_*, g_scale, y   as for moe_expert_ffn
 *   topk_idx, topk_w          [T, k] as from moe_route_topk
 *   workspace                 >= moe_expert_ffn_workspace_size(T,H,I,E,k)
 *                             bytes, owned by the caller (h [T*k, I] bf16 and
 *                             o [T*k, H] fp16), contents unspecified
 * Shapes and envelope: those of moe_expert_ffn, plus T*k*ceil(H/16) below
 * 2^31 workgroups.  For measurement beside the reuse path; moe_step is the
 * product path.
 */
moe_status moe_expert_ffn_per_route(const uint16_t* x,
                                    const uint8_t* w_gate, const uint8_t* s_gate,
                                    const uint8_t* w_up, const uint8_t* s_up,
                                    const uint8_t* w_down, const uint8_t* s_down,
                                    const float* g_scale,
                                    const int32_t* topk_idx, const float* topk_w,
                                    int T, int H, int I, int E, int k,
                                    void* workspace, size_t workspace_bytes,
                                    uint16_t* y, void* stream);

/*
 * moe_step_noalloc — moe_step (moe_step_packed when `packed` is not NULL)
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It takes
 * no workspace argument: its workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (8 MiB) inside the library, one copy per GPU the
 * library runs on, held until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine).
 *   Arguments and outputs: as moe_step / moe_step_packed, without workspace
 *   and workspace_bytes; outputs bit for bit those of moe_step with a
 *   workspace of its own.
 *   Limit: moe_step_workspace_size(T,H,I,E,k) <= MOE_NOALLOC_SCRATCH_BYTES
 *   (at H = 2048, I = 512, E = 512, k = 10: up to 163 tokens), else
 *   MOE_ERR_SCRATCH_TOO_SMALL and nothing is launched; every other check as
 *   for moe_step, before any launch.
 *   The scratch needs no clearing: like moe_step's workspace, nothing in it
 *   is read before the same call wrote it.  Every call on one GPU shares that
 *   GPU's array, so calls that overlap on one GPU (on different streams, or
 *   from different host threads) race; serialise them.  `stream` must belong
 *   to the current device.  The first call on each device looks up the
 *   array's device address (a host-side query, not a launch); make that
 *   first call outside graph capture.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
moe_status moe_step_noalloc(const uint16_t* x, const float* logits, const float* bias,
                            const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up,
                            const uint8_t* w_down, const uint8_t* s_down,
                            const float* g_scale, const uint8_t* packed,
                            int T, int H, int I, int E, int k,
                            int32_t* topk_idx, float* topk_w,
                            int32_t* expert_count, int32_t* expert_offset,
                            int32_t* active_experts, int32_t* n_active,
                            int32_t* route_src, int32_t* route_pos,
                            uint16_t* y, void* stream);

/* Static English description of a status code (never NULL). */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MOE_EXPERT_AMD_MOE_H */
