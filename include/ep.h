/*
 * ep.h - MoE token dispatch / combine on one MI355X (gfx950): C ABI.
 *
 * The pages this library follows describe DeepSeek's DeepEP:
 *   [P1] "DeepSeek 开源周第二弹：DeepEP —— 首个 MoE 模型训练和推理的 EP 通信库"
 *        (m.youleyou.com), sections "DeepEP 的核心功能" and
 *        "DeepEP 的常规内核和低延迟内核";
 *   [P4] the DeepEP article on deepseek.csdn.net, sections
 *        "使用示例 › MoE 训练中的应用" and "使用示例 › 推理解码阶段的应用";
 *   [P5] "deepseek-ai/DeepEP" (agentlenshq.com), section "典型工作流程".
 * There, dispatch(x, topk_idx, topk_weights, num_experts) sends every token
 * to the experts it is routed to and returns the received rows plus a
 * handle; combine uses the handle to reduce the expert outputs back to the
 * tokens.  On one GPU all experts are resident, so "send" becomes a
 * permutation into an expert-major receive buffer in the same HBM, and the
 * handle is the routing layout below.  The pages' single dispatch call is
 * split into ep_dispatch_layout (routing metadata) and ep_dispatch (the
 * data movement), and is also offered whole as ep_layout_dispatch;
 * ep_combine is the reduction.
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers to contiguous row-major
 *     memory owned by the caller.  The library allocates nothing, keeps no
 *     state between calls (a step plan lives in the caller's storage) and
 *     is safe to call from several host threads.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises with
 *     the host.  Results are valid once the stream reaches that point.
 *   - Arguments are checked on the host before anything is launched.  On
 *     an error the call returns a non-zero ep_status and has enqueued
 *     nothing.  EP_ERR_HIP means a launch was refused by the runtime.
 *   - Notation: T tokens, K experts per token (top-k), E experts, H hidden
 *     channels, R = T*K receive rows, G = H/128 scale groups per row.
 *   - Expert ids outside [0, E) in topk_idx (for example -1) mark an entry
 *     as masked: it is not counted, has slot -1, and dispatch and combine
 *     skip it.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size */
  EP_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle */
  EP_ERR_HIP = 3          /* the HIP runtime refused a launch */
} ep_status;

typedef enum {
  /* OCP E4M3FN bytes [R, H] plus one binary32 scale per 128 channels
   * [R, G]; requires H % 128 == 0. */
  EP_RECV_FP8_E4M3_G128 = 0,
  /* the token's BF16 bits copied unchanged [R, H]; requires H % 8 == 0. */
  EP_RECV_BF16 = 1
} ep_recv_format;

#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 32

/* Human-readable name of a status code (static storage). */
const char* ep_status_string(int status);

/* Bytes of device workspace ep_dispatch_layout, ep_dispatch_layout_padded
 * and ep_layout_dispatch (and their _i64 forms) need for this shape: 0 up
 * to 65536 entries (T*K), which one launch handles; beyond, (E+1) int32
 * per 4096-entry chunk.  Pure host function. */
size_t ep_layout_workspace_bytes(int64_t num_tokens, int32_t top_k, int32_t num_experts);

/*
 * ep_dispatch_layout - routing layout of one dispatch.
 *
 * Defines the handle of [P4 "使用示例 › MoE 训练中的应用"] and the
 * per-expert received count of [P4 "使用示例 › 推理解码阶段的应用"].  The
 * pages leave the order inside an expert open; here it is ascending token
 * index (ascending k inside a token), which makes every output
 * deterministic:
 *
 *   tokens_per_expert[e] = #{(t,k) : topk_idx[t,k] == e}
 *   expert_offset[0] = 0, expert_offset[e+1] = expert_offset[e] + tokens_per_expert[e]
 *   slot[t,k] = expert_offset[e] + #{(t',k') before (t,k) in (t,k) order with expert e}
 *               (-1 for a masked entry)
 *   src_token[slot[t,k]] = t, and src_token[r] = -1 for r >= expert_offset[E]
 *
 * topk_idx          int32 [T, K] in
 * tokens_per_expert int32 [E]    out
 * expert_offset     int32 [E+1]  out (expert_offset[E] = number of unmasked entries)
 * slot              int32 [T, K] out (the handle's forward map)
 * src_token         int32 [T*K]  out (the handle's inverse map)
 * workspace         device scratch of >= ep_layout_workspace_bytes(T, K, E)
 *                   bytes, 16-byte aligned (may be NULL when that is 0);
 *                   its contents are clobbered.
 * Requirements: T >= 0, 1 <= K <= EP_MAX_TOPK, 1 <= E <= EP_MAX_EXPERTS,
 * T*K <= 2^22, int32 arrays 4-byte aligned.  T == 0 writes zero counts and
 * offsets.  topk_idx aligned to 16 bytes takes a faster load path.
 */
ep_status ep_dispatch_layout(const int32_t* topk_idx, int64_t num_tokens, int32_t top_k,
                             int32_t num_experts, int32_t* tokens_per_expert,
                             int32_t* expert_offset, int32_t* slot, int32_t* src_token,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * ep_dispatch_layout_padded - the low-latency layout: a fixed capacity of
 * rows per expert.
 *
 * [P4 "使用示例 › 推理解码阶段的应用"]: the low-latency buffer holds
 * num_max_tokens rows for every expert (num_max_tokens * hidden *
 * num_experts) and the low-latency dispatch reports recv_expert_count.
 * Expert e owns receive rows e*capacity .. e*capacity + capacity - 1; an
 * entry's rank inside its expert is the same stable (t, k) rank as in
 * ep_dispatch_layout:
 *   slot[t,k] = e*capacity + rank   if rank < capacity, else -1 (dropped;
 *               the pages give no overflow rule) and -1 for masked entries
 *   recv_expert_count[e] = min(#{(t,k) : topk_idx[t,k] == e}, capacity)
 *   src_token[e*capacity + i] = token of that row for i < recv_expert_count[e];
 *                               the unused rows of an expert are not written
 * With capacity >= T and distinct experts per token nothing is dropped.
 * ep_dispatch and ep_combine take this slot unchanged; their receive / expert
 * buffers then have E*capacity rows.
 *
 * recv_expert_count int32 [E] out;  slot int32 [T, K] out;
 * src_token int32 [E*capacity] out;  workspace as for ep_dispatch_layout
 * (same size function).  Requirements: capacity >= 1, E*capacity < 2^31,
 * otherwise as for ep_dispatch_layout.
 */
ep_status ep_dispatch_layout_padded(const int32_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                    int32_t num_experts, int32_t capacity, int32_t* recv_expert_count,
                                    int32_t* slot, int32_t* src_token, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * The same two layout calls with int64 expert ids (the index type routers
 * usually produce, e.g. a top-k over gate scores): identical results, the
 * ids read as 64-bit values (8-byte aligned).  An id outside [0, E) is
 * masked, whatever its width.
 */
ep_status ep_dispatch_layout_i64(const int64_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                 int32_t num_experts, int32_t* tokens_per_expert, int32_t* expert_offset,
                                 int32_t* slot, int32_t* src_token, void* workspace, size_t workspace_bytes,
                                 void* stream);
ep_status ep_dispatch_layout_padded_i64(const int64_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                        int32_t num_experts, int32_t capacity, int32_t* recv_expert_count,
                                        int32_t* slot, int32_t* src_token, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * ep_dispatch - copy every token into its K receive rows.
 *
 * [P1 "DeepEP 的常规内核和低延迟内核"]: dispatch moves tokens to their
 * experts in FP8.  The per-128-channel granularity and the scale formula
 * are not given by the pages; this library uses, per token t and group g
 * of 128 channels:
 *   a = max |x[t,c]|,  s = RN32(a / 448)  (s = 1 if a == 0; s = 2^-126 if
 *   a / 448 would be below 2^-126),
 *   q[c] = E4M3FN_RNE(RN32(x[t,c] / s))   (one correctly rounded division)
 * and for each unmasked k with r = slot[t,k]:
 *   recv_x[r, :] = q,  recv_scale[r, g] = s,  recv_weight[r] = topk_weights[t,k].
 * With EP_RECV_BF16, recv_x[r, :] = x[t, :] bit for bit and recv_scale is
 * unused (may be NULL).
 *
 * x            bf16 bits [T, H] in, 16-byte aligned
 * slot         int32 [T, K] from ep_dispatch_layout
 * topk_weights float32 [T, K] or NULL (then recv_weight must be NULL)
 * recv_x       [rows, H] out: uint8 (FP8) or bf16 bits, 16-byte aligned;
 *              rows = T*K for ep_dispatch_layout's slot, E*capacity for
 *              ep_dispatch_layout_padded's
 * recv_scale   float32 [rows, G] out (FP8 only), 4-byte aligned
 * recv_weight  float32 [rows] out or NULL
 * Rows no entry maps to are left untouched.  Requirements: H > 0,
 * H % 128 == 0 for FP8, H % 8 == 0 for BF16, 1 <= K <= EP_MAX_TOPK,
 * T*K <= 2^22, T*H < 2^34.
 */
ep_status ep_dispatch(const void* x, int64_t num_tokens, int32_t hidden, int32_t top_k,
                      const int32_t* slot, const float* topk_weights, int32_t format,
                      void* recv_x, float* recv_scale, float* recv_weight, void* stream);

/*
 * ep_layout_dispatch - layout and dispatch in one call, the shape of the
 * pages' dispatch call, which takes the tokens with their routing and
 * returns the received rows together with the handle ([P4 "使用示例 › MoE
 * 训练中的应用"]), or, with capacity > 0, fills per-expert buffers and
 * reports per-expert counts ([P4 "使用示例 › 推理解码阶段的应用"]).
 *
 * Writes exactly what ep_dispatch_layout (capacity == 0) or
 * ep_dispatch_layout_padded (capacity > 0) followed by ep_dispatch would
 * write, bit for bit.  Up to 3072 entries (T*K) this is one kernel launch
 * built for the decode sizes, where launch latency dominates; up to 65536
 * entries another single launch, in which each workgroup lays out and
 * dispatches its own tokens (when its share fits: at most 8 FP8 or 14 BF16
 * work items per lane of 1024, at most one entry per lane, and the
 * layout's LDS within the 160 KB of a workgroup, e.g. 4096 tokens of hidden
 * 7168 at top-8; else as beyond); beyond, the same launches as the
 * separate calls.
 *
 * topk_idx, tokens_per_expert, slot, src_token, workspace: as for
 *   ep_dispatch_layout (capacity == 0) or ep_dispatch_layout_padded
 *   (capacity > 0, where tokens_per_expert receives recv_expert_count);
 * expert_offset int32 [E+1] out for capacity == 0; unused and may be NULL
 *   for capacity > 0;
 * x, topk_weights, format, recv_x, recv_scale, recv_weight: as for
 *   ep_dispatch, with rows = T*K (capacity == 0) or E*capacity.
 * Requirements: the union of those calls' requirements.
 */
ep_status ep_layout_dispatch(const int32_t* topk_idx, const void* x, const float* topk_weights,
                             int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                             int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                             int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                             float* recv_scale, float* recv_weight, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ep_layout_dispatch with int64 expert ids (8-byte aligned); otherwise identical. */
ep_status ep_layout_dispatch_i64(const int64_t* topk_idx, const void* x, const float* topk_weights,
                                 int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                 int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                                 int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                                 float* recv_scale, float* recv_weight, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * ep_layout_dispatch_noalloc - ep_layout_dispatch for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same results bit for bit, and no allocation of any kind.
 *
 * The layout's per-chunk histograms (the only scratch, used beyond 65536
 * entries) live in a device array inside the library of
 * EP_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held until the process
 * ends.  Shapes whose histograms do not fit, ep_layout_workspace_bytes(T,
 * K, E) > EP_NOALLOC_SCRATCH_BYTES (e.g. beyond 1,044,480 entries at 1024
 * experts, or 4,177,920 at 256), return EP_ERR_UNSUPPORTED before anything
 * is launched.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from threads without
 * ordering) race on it and must be serialised by the caller, e.g. by
 * issuing them on one stream.  No part of the array needs clearing between
 * calls.  The first call on a device looks up the array's address there
 * (EP_ERR_HIP if the runtime cannot give it).
 */
#define EP_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
ep_status ep_layout_dispatch_noalloc(const int32_t* topk_idx, const void* x, const float* topk_weights,
                                     int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                     int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                                     int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                                     float* recv_scale, float* recv_weight, void* stream);

/*
 * ep_combine - reduce each token's K expert outputs back to the token.
 *
 * [P5 "典型工作流程"]: combine reduces the expert outputs back to the
 * source; [P1 "DeepEP 的常规内核和低延迟内核"]: in BF16.  Arithmetic
 * (not fixed by the pages): binary32, ascending k, product rounded before
 * the add (no fused multiply-add), starting from +0.0, result rounded once
 * to BF16 (round to nearest even):
 *   acc = +0.0; for k with r = slot[t,k] >= 0:
 *       acc = RN32(acc + RN32(topk_weights[t,k] * y[r,c]))
 *   out[t,c] = BF16_RNE(acc)
 *
 * y            bf16 bits [rows, H] in (receive-row order; rows as for
 *              ep_dispatch), 16-byte aligned
 * slot         int32 [T, K] from ep_dispatch_layout or _padded
 * topk_weights float32 [T, K]
 * out          bf16 bits [T, H] out, 16-byte aligned; must not overlap y
 * Requirements: H > 0, H % 8 == 0, 1 <= K <= EP_MAX_TOPK, T*K <= 2^22,
 * T*H < 2^34.
 */
ep_status ep_combine(const void* y, const int32_t* slot, const float* topk_weights,
                     int64_t num_tokens, int32_t hidden, int32_t top_k, void* out,
                     void* stream);

/*
 * ep_step_plan - one MoE step's two launches with their arguments checked
 * once.
 *
 * [P4 "使用示例 › 推理解码阶段的应用"] runs dispatch, the expert GEMMs and
 * combine once per decoding step, on buffers that stay the same from step
 * to step.  A plan records the arguments of one ep_layout_dispatch call
 * (int32 or int64 ids) and of the ep_combine call on the same tokens,
 * checked by ep_step_plan_init, so that each step's launches take one
 * pointer each.  At decode sizes the host cost of a call (the argument
 * checks, and marshalling many arguments from an interpreter) is of the
 * order of the kernels' few microseconds of GPU time.
 *
 * The plan is plain data in caller-owned storage: the library allocates
 * nothing, and a plan may be copied.  It records pointers only: the
 * buffers must outlive its use, and their contents may change from step
 * to step.  A plan's launches behave exactly as the calls it records.
 */
typedef struct {
  uint64_t opaque[32];
} ep_step_plan;

/*
 * ep_step_plan_init - check and record a step's arguments.
 *
 * id_bytes: 4 for int32 topk_idx, 8 for int64 (8-byte aligned).  The
 * arguments from topk_idx to workspace_bytes, and stream, are those of
 * ep_layout_dispatch; y and out are those of ep_combine, whose slot,
 * topk_weights, T, H and K are the ones given here.  topk_weights feeds
 * combine, and the dispatch only when recv_weight is given.  y and out may
 * both be NULL for a plan that only lays out and dispatches.
 * Returns what ep_layout_dispatch or ep_combine would return for a bad
 * argument (EP_ERR_INVALID_ARG also for a NULL or misaligned plan or
 * another id_bytes); a plan whose init failed launches nothing (its calls
 * return EP_ERR_INVALID_ARG).  Pure host function.
 */
ep_status ep_step_plan_init(ep_step_plan* plan, const void* topk_idx, int32_t id_bytes, const void* x,
                            const float* topk_weights, int64_t num_tokens, int32_t hidden, int32_t top_k,
                            int32_t num_experts, int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                            int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                            float* recv_scale, float* recv_weight, void* workspace, size_t workspace_bytes,
                            const void* y, void* out, void* stream);

/* The plan's ep_layout_dispatch launch. */
ep_status ep_step_plan_layout_dispatch(const ep_step_plan* plan);

/* The plan's ep_combine launch; EP_ERR_INVALID_ARG for a plan without y
 * and out (unless T == 0, where there is nothing to reduce). */
ep_status ep_step_plan_combine(const ep_step_plan* plan);

/*
 * ep_dispatch_backward - gradient of dispatch w.r.t. the tokens.
 *
 * [P5 "典型工作流程"] lists backward helpers beside combine; the pages give
 * no arithmetic.  Dispatch copies token t into K rows, so its gradient sums
 * the K rows' gradients (an FP8 cast is passed straight through).  Same
 * arithmetic as ep_combine with every weight 1:
 *   grad_x[t,c] = BF16_RNE(+0.0 + grad_recv[slot[t,0],c] + ... ), binary32,
 *   ascending k, masked entries skipped.
 * grad_recv bf16 [rows, H] in; slot int32 [T, K]; grad_x bf16 [T, H] out.
 * Requirements as for ep_combine.
 */
ep_status ep_dispatch_backward(const void* grad_recv, const int32_t* slot, int64_t num_tokens,
                               int32_t hidden, int32_t top_k, void* grad_x, void* stream);

/*
 * ep_combine_backward - gradients of combine w.r.t. the expert outputs y
 * and the routing weights ([P5 "典型工作流程"], backward helpers):
 *   grad_y[slot[t,k], c] = BF16_RNE(RN32(topk_weights[t,k] * grad_out[t,c]))
 *   grad_w[t,k] = sum_c grad_out[t,c] * y[slot[t,k], c]      (binary32)
 * Every product of two BF16 values is exact in binary32; the sum is taken
 * in a fixed order (so results are reproducible run to run), in which
 * each product passes through at most 7 + ceil(log2(H/8)) rounded binary32
 * additions: the 8 products of each 8-channel vector are added in channel
 * order into +0.0, then the H/8 vector sums as a binary tree.  grad_w is
 * therefore within (7 + ceil(log2(H/8))) * 2^-24 * (1 + 2^-16) *
 * sum_c |grad_out[t,c] * y[slot[t,k], c]| of the exact dot product (plus
 * H * 2^-150 where products fall below the normal binary32 range).
 * Masked entries get grad_w = +0.0 and no grad_y row; other grad_y rows are
 * left untouched.
 * grad_out bf16 [T, H]; y bf16 [rows, H] (may be NULL when grad_w is NULL);
 * slot int32 [T, K]; topk_weights float32 [T, K]; grad_y bf16 [rows, H]
 * out; grad_w float32 [T, K] out or NULL.
 * Requirements: H % 8 == 0, H <= 8192 (one workgroup per token), otherwise
 * as for ep_combine.
 */
ep_status ep_combine_backward(const void* grad_out, const void* y, const int32_t* slot,
                              const float* topk_weights, int64_t num_tokens, int32_t hidden, int32_t top_k,
                              void* grad_y, float* grad_w, void* stream);

/*
 * ep_cast_fp8_e4m3 - the binary32 -> E4M3FN conversion ep_dispatch uses,
 * applied elementwise: out[i] = E4M3FN_RNE_satfinite(in[i]).  Magnitudes
 * beyond 448 saturate to +-448; NaN inputs are outside the contract.
 * Exposed so the conversion can be checked exhaustively against its
 * definition (OCP 8-bit floating point specification v1.0).
 * in float32 [n], out uint8 [n]; 0 <= n < 2^33; both 16-byte aligned.
 */
ep_status ep_cast_fp8_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
