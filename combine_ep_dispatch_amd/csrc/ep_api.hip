// C ABI of the MoE dispatch/combine library: argument checks, then kernel
// launches on the caller's stream.  See include/ep.h for the contract.

#include "../../include/ep.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ep_internal.h"

#define EP_API extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest T*K handled: bounds the per-key scan over chunks in the layout's
// second pass (at most 1024 chunks of 4096 entries).
constexpr int64_t kMaxRows = int64_t(1) << 22;

// Largest T*H handled by dispatch, combine and their backward: their
// kernels launch T*H/16 or T*H/8 work items (the per-token backward
// workgroups at most T*(H/8 + 63)).  Below 2^31 items the 32-bit item
// counts and grid arithmetic are exact and every launch is in range.
constexpr int64_t kMaxElems = int64_t(1) << 34;

// Largest n handled by ep_cast_fp8_e4m3 (n/4 work items, below 2^31).
constexpr int64_t kMaxCast = int64_t(1) << 33;

ep_status from_hip(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

constexpr int kMaxDevices = 64;

ep_status check_common(int64_t T, int32_t K) {
  if (T < 0 || K < 1) return EP_ERR_INVALID_ARG;
  if (K > EP_MAX_TOPK) return EP_ERR_UNSUPPORTED;
  if (T * K >= (int64_t(1) << 31)) return EP_ERR_INVALID_ARG;
  if (T * K > kMaxRows) return EP_ERR_UNSUPPORTED;
  return EP_OK;
}

// Checks of the layout arguments (capacity 0: packed layout with offsets;
// capacity > 0: padded layout, offsets unused).
// id_bytes: width of one expert id (4 or 8); the ids must be aligned to it.
ep_status check_layout(const void* topk_idx, size_t id_bytes, int64_t T, int32_t K, int32_t E, int32_t capacity,
                       const int32_t* counts, const int32_t* offsets, const int32_t* slot, const int32_t* src,
                       const void* workspace, size_t workspace_bytes) {
  ep_status st = check_common(T, K);
  if (st != EP_OK) return st;
  if (E < 1 || capacity < 0) return EP_ERR_INVALID_ARG;
  if (E > EP_MAX_EXPERTS) return EP_ERR_UNSUPPORTED;
  if (!counts || !aligned(counts, 4)) return EP_ERR_INVALID_ARG;
  if (capacity == 0) {
    if (!offsets || !aligned(offsets, 4)) return EP_ERR_INVALID_ARG;
  } else {
    if (static_cast<int64_t>(E) * capacity >= (int64_t(1) << 31)) return EP_ERR_INVALID_ARG;
    if (!src || !aligned(src, 4)) return EP_ERR_INVALID_ARG;
  }
  const int64_t rows = T * K;
  if (rows > 0) {
    if (!topk_idx || !slot || !src) return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, id_bytes) || !aligned(slot, 4) || !aligned(src, 4)) return EP_ERR_INVALID_ARG;
  }
  const size_t need = ep::layout_workspace_bytes(rows, E);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return EP_ERR_INVALID_ARG;
  return EP_OK;
}

// Checks of the dispatch arguments other than slot; the buffers are only
// checked when there are tokens.
ep_status check_dispatch(const void* x, int64_t T, int32_t H, int32_t K, const float* topk_weights, int32_t format,
                         const void* recv_x, const float* recv_scale, const float* recv_weight) {
  ep_status st = check_common(T, K);
  if (st != EP_OK) return st;
  if (H <= 0) return EP_ERR_INVALID_ARG;
  if (format != EP_RECV_FP8_E4M3_G128 && format != EP_RECV_BF16) return EP_ERR_INVALID_ARG;
  if (format == EP_RECV_FP8_E4M3_G128 && H % 128 != 0) return EP_ERR_INVALID_ARG;
  if (H % 8 != 0) return EP_ERR_INVALID_ARG;
  if (recv_weight != nullptr && topk_weights == nullptr) return EP_ERR_INVALID_ARG;
  if (T * H >= kMaxElems) return EP_ERR_UNSUPPORTED;
  if (T == 0) return EP_OK;
  if (!x || !recv_x) return EP_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(recv_x, 16)) return EP_ERR_INVALID_ARG;
  if (topk_weights && !aligned(topk_weights, 4)) return EP_ERR_INVALID_ARG;
  if (recv_weight && !aligned(recv_weight, 4)) return EP_ERR_INVALID_ARG;
  if (format == EP_RECV_FP8_E4M3_G128 && (!recv_scale || !aligned(recv_scale, 4))) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

}  // namespace

namespace ep {

int device_cu_count() {
  // threads that race to fill an entry all store the same value
  static std::atomic<int> cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace ep

EP_API const char* ep_status_string(int status) {
  switch (status) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
    case EP_ERR_HIP: return "EP_ERR_HIP";
    default: return "EP_ERR_UNKNOWN";
  }
}

EP_API size_t ep_layout_workspace_bytes(int64_t num_tokens, int32_t top_k, int32_t num_experts) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || num_experts > EP_MAX_EXPERTS) return 0;
  return ep::layout_workspace_bytes(num_tokens * top_k, num_experts);
}

namespace {

template <typename Idx>
ep_status dispatch_layout(const Idx* topk_idx, int64_t num_tokens, int32_t top_k, int32_t num_experts,
                          int32_t* tokens_per_expert, int32_t* expert_offset, int32_t* slot, int32_t* src_token,
                          void* workspace, size_t workspace_bytes, void* stream) {
  ep_status st = check_layout(topk_idx, sizeof(Idx), num_tokens, top_k, num_experts, 0, tokens_per_expert,
                              expert_offset, slot, src_token, workspace, workspace_bytes);
  if (st != EP_OK) return st;
  return from_hip(ep::launch_layout(topk_idx, static_cast<int32_t>(num_tokens * top_k), top_k, num_experts, 0,
                                    tokens_per_expert, expert_offset, slot, src_token, workspace,
                                    static_cast<hipStream_t>(stream)));
}

template <typename Idx>
ep_status dispatch_layout_padded(const Idx* topk_idx, int64_t num_tokens, int32_t top_k, int32_t num_experts,
                                 int32_t capacity, int32_t* recv_expert_count, int32_t* slot, int32_t* src_token,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  ep_status st = check_common(num_tokens, top_k);
  if (st != EP_OK) return st;
  if (capacity < 1) return EP_ERR_INVALID_ARG;
  st = check_layout(topk_idx, sizeof(Idx), num_tokens, top_k, num_experts, capacity, recv_expert_count, nullptr,
                    slot, src_token, workspace, workspace_bytes);
  if (st != EP_OK) return st;
  return from_hip(ep::launch_layout(topk_idx, static_cast<int32_t>(num_tokens * top_k), top_k, num_experts,
                                    capacity, recv_expert_count, nullptr, slot, src_token, workspace,
                                    static_cast<hipStream_t>(stream)));
}

}  // namespace

EP_API ep_status ep_dispatch_layout(const int32_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                    int32_t num_experts, int32_t* tokens_per_expert, int32_t* expert_offset,
                                    int32_t* slot, int32_t* src_token, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return dispatch_layout(topk_idx, num_tokens, top_k, num_experts, tokens_per_expert, expert_offset, slot,
                         src_token, workspace, workspace_bytes, stream);
}

EP_API ep_status ep_dispatch_layout_i64(const int64_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                        int32_t num_experts, int32_t* tokens_per_expert, int32_t* expert_offset,
                                        int32_t* slot, int32_t* src_token, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return dispatch_layout(topk_idx, num_tokens, top_k, num_experts, tokens_per_expert, expert_offset, slot,
                         src_token, workspace, workspace_bytes, stream);
}

EP_API ep_status ep_dispatch_layout_padded(const int32_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                           int32_t num_experts, int32_t capacity, int32_t* recv_expert_count,
                                           int32_t* slot, int32_t* src_token, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return dispatch_layout_padded(topk_idx, num_tokens, top_k, num_experts, capacity, recv_expert_count, slot,
                                src_token, workspace, workspace_bytes, stream);
}

EP_API ep_status ep_dispatch_layout_padded_i64(const int64_t* topk_idx, int64_t num_tokens, int32_t top_k,
                                               int32_t num_experts, int32_t capacity, int32_t* recv_expert_count,
                                               int32_t* slot, int32_t* src_token, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  return dispatch_layout_padded(topk_idx, num_tokens, top_k, num_experts, capacity, recv_expert_count, slot,
                                src_token, workspace, workspace_bytes, stream);
}

EP_API ep_status ep_dispatch(const void* x, int64_t num_tokens, int32_t hidden, int32_t top_k,
                             const int32_t* slot, const float* topk_weights, int32_t format, void* recv_x,
                             float* recv_scale, float* recv_weight, void* stream) {
  ep_status st = check_dispatch(x, num_tokens, hidden, top_k, topk_weights, format, recv_x, recv_scale, recv_weight);
  if (st != EP_OK) return st;
  if (num_tokens == 0) return EP_OK;
  if (!slot || !aligned(slot, 4)) return EP_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t T = static_cast<int32_t>(num_tokens);
  if (format == EP_RECV_FP8_E4M3_G128)
    return from_hip(ep::launch_dispatch_fp8(static_cast<const uint16_t*>(x), T, hidden, top_k, slot,
                                            topk_weights, static_cast<uint8_t*>(recv_x), recv_scale,
                                            recv_weight, s));
  return from_hip(ep::launch_dispatch_bf16(static_cast<const uint16_t*>(x), T, hidden, top_k, slot,
                                           topk_weights, static_cast<uint16_t*>(recv_x), recv_weight, s));
}

namespace {

template <typename Idx>
ep_status check_layout_dispatch(const Idx* topk_idx, const void* x, const float* topk_weights, int64_t num_tokens,
                                int32_t hidden, int32_t top_k, int32_t num_experts, int32_t capacity,
                                int32_t format, const int32_t* tokens_per_expert, const int32_t* expert_offset,
                                const int32_t* slot, const int32_t* src_token, const void* recv_x,
                                const float* recv_scale, const float* recv_weight, const void* workspace,
                                size_t workspace_bytes) {
  ep_status st = check_layout(topk_idx, sizeof(Idx), num_tokens, top_k, num_experts, capacity, tokens_per_expert,
                              capacity == 0 ? expert_offset : nullptr, slot, src_token, workspace,
                              workspace_bytes);
  if (st != EP_OK) return st;
  return check_dispatch(x, num_tokens, hidden, top_k, topk_weights, format, recv_x, recv_scale, recv_weight);
}

template <typename Idx>
ep_status layout_dispatch(const Idx* topk_idx, const void* x, const float* topk_weights, int64_t num_tokens,
                          int32_t hidden, int32_t top_k, int32_t num_experts, int32_t capacity, int32_t format,
                          int32_t* tokens_per_expert, int32_t* expert_offset, int32_t* slot, int32_t* src_token,
                          void* recv_x, float* recv_scale, float* recv_weight, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const ep_status st = check_layout_dispatch(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts,
                                             capacity, format, tokens_per_expert, expert_offset, slot, src_token,
                                             recv_x, recv_scale, recv_weight, workspace, workspace_bytes);
  if (st != EP_OK) return st;
  return from_hip(ep::launch_layout_dispatch(
      topk_idx, static_cast<const uint16_t*>(x), topk_weights, static_cast<int32_t>(num_tokens), hidden, top_k,
      num_experts, capacity, format == EP_RECV_FP8_E4M3_G128, tokens_per_expert,
      capacity == 0 ? expert_offset : nullptr, slot, src_token, recv_x, recv_scale, recv_weight, workspace,
      static_cast<hipStream_t>(stream)));
}

}  // namespace

EP_API ep_status ep_layout_dispatch(const int32_t* topk_idx, const void* x, const float* topk_weights,
                                    int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                    int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                                    int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                                    float* recv_scale, float* recv_weight, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return layout_dispatch(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity, format,
                         tokens_per_expert, expert_offset, slot, src_token, recv_x, recv_scale, recv_weight,
                         workspace, workspace_bytes, stream);
}

EP_API ep_status ep_layout_dispatch_i64(const int64_t* topk_idx, const void* x, const float* topk_weights,
                                        int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                        int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                                        int32_t* expert_offset, int32_t* slot, int32_t* src_token, void* recv_x,
                                        float* recv_scale, float* recv_weight, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return layout_dispatch(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity, format,
                         tokens_per_expert, expert_offset, slot, src_token, recv_x, recv_scale, recv_weight,
                         workspace, workspace_bytes, stream);
}

// ---- the allocation-free form of ep_layout_dispatch ------------------------
//
// The only device scratch any kernel here uses is the per-chunk histograms of
// the two-launch layout (beyond 65536 entries).  ep_layout_dispatch_noalloc
// keeps them in this file-scope array instead of a caller's workspace.  Each
// GPU the library runs on holds its own copy (at its own address) until the
// process ends.  Host code never passes the array's name to a kernel: in host
// code it is a stand-in, not a device address.  The device address comes from
// hipGetSymbolAddress, taken once per device with that device current.

namespace {

constexpr size_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;  // (E+1) int32 per 4096-entry chunk
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch (nullptr if the runtime cannot
// give it).
void* device_scratch() {
  static std::atomic<void*> ptrs[kMaxDevices] = {};
  static std::mutex once;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(once);
  p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

// A stand-in for the scratch during the argument checks (aligned, of any
// size, never dereferenced); the scratch's own limit is checked after them.
void* const kCheckOnly = reinterpret_cast<void*>(uintptr_t(256));

}  // namespace

EP_API ep_status ep_layout_dispatch_noalloc(const int32_t* topk_idx, const void* x, const float* topk_weights,
                                            int64_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                            int32_t capacity, int32_t format, int32_t* tokens_per_expert,
                                            int32_t* expert_offset, int32_t* slot, int32_t* src_token,
                                            void* recv_x, float* recv_scale, float* recv_weight, void* stream) {
  ep_status st = check_layout_dispatch(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity,
                                       format, tokens_per_expert, expert_offset, slot, src_token, recv_x,
                                       recv_scale, recv_weight, kCheckOnly, SIZE_MAX);
  if (st != EP_OK) return st;
  const size_t need = ep::layout_workspace_bytes(num_tokens * top_k, num_experts);
  if (need > kScratchBytes) return EP_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (ws == nullptr) return EP_ERR_HIP;
  }
  return layout_dispatch(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity, format,
                         tokens_per_expert, expert_offset, slot, src_token, recv_x, recv_scale, recv_weight, ws,
                         ws != nullptr ? kScratchBytes : 0, stream);
}

namespace {

ep_status check_combine(const void* y, const int32_t* slot, const float* topk_weights, int64_t num_tokens,
                        int32_t hidden, int32_t top_k, const void* out) {
  ep_status st = check_common(num_tokens, top_k);
  if (st != EP_OK) return st;
  if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARG;
  if (num_tokens * hidden >= kMaxElems) return EP_ERR_UNSUPPORTED;
  if (num_tokens == 0) return EP_OK;
  if (!y || !slot || !topk_weights || !out) return EP_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot, 4) || !aligned(topk_weights, 4))
    return EP_ERR_INVALID_ARG;
  return EP_OK;
}

}  // namespace

EP_API ep_status ep_combine(const void* y, const int32_t* slot, const float* topk_weights, int64_t num_tokens,
                            int32_t hidden, int32_t top_k, void* out, void* stream) {
  const ep_status st = check_combine(y, slot, topk_weights, num_tokens, hidden, top_k, out);
  if (st != EP_OK || num_tokens == 0) return st;
  return from_hip(ep::launch_combine(static_cast<const uint16_t*>(y), slot, topk_weights,
                                     static_cast<int32_t>(num_tokens), hidden, top_k,
                                     static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

// ---- step plans --------------------------------------------------------------
//
// The arguments of one ep_layout_dispatch call and one ep_combine call,
// checked once, kept in the caller's ep_step_plan storage.  `magic` is set
// last, and only when every check passed, so a plan whose init failed (or
// that was never initialised) launches nothing.

namespace {

constexpr uint32_t kPlanMagic = 0x45505350u;  // "EPSP"

struct Plan {
  uint32_t magic;
  int32_t id_bytes;
  int32_t hidden, top_k, num_experts, capacity, format, has_combine;
  int64_t num_tokens;
  const void* topk_idx;
  const void* x;
  const float* topk_weights;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot;
  int32_t* src;
  void* recv_x;
  float* recv_scale;
  float* recv_weight;
  void* workspace;
  const void* y;
  void* out;
  void* stream;
};
static_assert(sizeof(Plan) <= sizeof(ep_step_plan), "plan storage");
static_assert(alignof(Plan) <= alignof(ep_step_plan), "plan alignment");

template <typename Idx>
ep_status plan_layout_dispatch(const Plan& p) {
  return from_hip(ep::launch_layout_dispatch(
      static_cast<const Idx*>(p.topk_idx), static_cast<const uint16_t*>(p.x), p.topk_weights,
      static_cast<int32_t>(p.num_tokens), p.hidden, p.top_k, p.num_experts, p.capacity,
      p.format == EP_RECV_FP8_E4M3_G128, p.counts, p.capacity == 0 ? p.offsets : nullptr, p.slot, p.src, p.recv_x,
      p.recv_scale, p.recv_weight, p.workspace, static_cast<hipStream_t>(p.stream)));
}

}  // namespace

EP_API ep_status ep_step_plan_init(ep_step_plan* plan, const void* topk_idx, int32_t id_bytes, const void* x,
                                   const float* topk_weights, int64_t num_tokens, int32_t hidden, int32_t top_k,
                                   int32_t num_experts, int32_t capacity, int32_t format,
                                   int32_t* tokens_per_expert, int32_t* expert_offset, int32_t* slot,
                                   int32_t* src_token, void* recv_x, float* recv_scale, float* recv_weight,
                                   void* workspace, size_t workspace_bytes, const void* y, void* out,
                                   void* stream) {
  if (plan == nullptr || !aligned(plan, alignof(ep_step_plan))) return EP_ERR_INVALID_ARG;
  Plan* p = reinterpret_cast<Plan*>(plan);
  p->magic = 0;
  if (id_bytes != 4 && id_bytes != 8) return EP_ERR_INVALID_ARG;
  ep_status st =
      id_bytes == 4
          ? check_layout_dispatch(static_cast<const int32_t*>(topk_idx), x, topk_weights, num_tokens, hidden,
                                  top_k, num_experts, capacity, format, tokens_per_expert, expert_offset, slot,
                                  src_token, recv_x, recv_scale, recv_weight, workspace, workspace_bytes)
          : check_layout_dispatch(static_cast<const int64_t*>(topk_idx), x, topk_weights, num_tokens, hidden,
                                  top_k, num_experts, capacity, format, tokens_per_expert, expert_offset, slot,
                                  src_token, recv_x, recv_scale, recv_weight, workspace, workspace_bytes);
  if (st != EP_OK) return st;
  const bool has_combine = y != nullptr || out != nullptr;
  if (has_combine) {
    st = check_combine(y, slot, topk_weights, num_tokens, hidden, top_k, out);
    if (st != EP_OK) return st;
  }
  *p = Plan{0,           id_bytes,     hidden, top_k,     num_experts,   capacity,   format,
            has_combine, num_tokens,   topk_idx, x,       topk_weights,  tokens_per_expert, expert_offset,
            slot,        src_token,    recv_x, recv_scale, recv_weight,  workspace,  y,
            out,         stream};
  p->magic = kPlanMagic;
  return EP_OK;
}

EP_API ep_status ep_step_plan_layout_dispatch(const ep_step_plan* plan) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr || p->magic != kPlanMagic) return EP_ERR_INVALID_ARG;
  return p->id_bytes == 4 ? plan_layout_dispatch<int32_t>(*p) : plan_layout_dispatch<int64_t>(*p);
}

EP_API ep_status ep_step_plan_combine(const ep_step_plan* plan) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr || p->magic != kPlanMagic) return EP_ERR_INVALID_ARG;
  if (p->num_tokens == 0) return EP_OK;  // as ep_combine: nothing to reduce
  if (!p->has_combine) return EP_ERR_INVALID_ARG;
  return from_hip(ep::launch_combine(static_cast<const uint16_t*>(p->y), p->slot, p->topk_weights,
                                     static_cast<int32_t>(p->num_tokens), p->hidden, p->top_k,
                                     static_cast<uint16_t*>(p->out), static_cast<hipStream_t>(p->stream)));
}

EP_API ep_status ep_dispatch_backward(const void* grad_recv, const int32_t* slot, int64_t num_tokens,
                                      int32_t hidden, int32_t top_k, void* grad_x, void* stream) {
  ep_status st = check_common(num_tokens, top_k);
  if (st != EP_OK) return st;
  if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARG;
  if (num_tokens * hidden >= kMaxElems) return EP_ERR_UNSUPPORTED;
  if (num_tokens == 0) return EP_OK;
  if (!grad_recv || !slot || !grad_x) return EP_ERR_INVALID_ARG;
  if (!aligned(grad_recv, 16) || !aligned(grad_x, 16) || !aligned(slot, 4)) return EP_ERR_INVALID_ARG;
  return from_hip(ep::launch_combine(static_cast<const uint16_t*>(grad_recv), slot, nullptr,
                                     static_cast<int32_t>(num_tokens), hidden, top_k,
                                     static_cast<uint16_t*>(grad_x), static_cast<hipStream_t>(stream)));
}

EP_API ep_status ep_combine_backward(const void* grad_out, const void* y, const int32_t* slot,
                                     const float* topk_weights, int64_t num_tokens, int32_t hidden, int32_t top_k,
                                     void* grad_y, float* grad_w, void* stream) {
  ep_status st = check_common(num_tokens, top_k);
  if (st != EP_OK) return st;
  if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARG;
  if (hidden > 8192) return EP_ERR_UNSUPPORTED;
  if (num_tokens * hidden >= kMaxElems) return EP_ERR_UNSUPPORTED;
  if (num_tokens == 0) return EP_OK;
  if (!grad_out || !slot || !topk_weights || !grad_y) return EP_ERR_INVALID_ARG;
  if (grad_w != nullptr && y == nullptr) return EP_ERR_INVALID_ARG;
  if (!aligned(grad_out, 16) || !aligned(grad_y, 16) || !aligned(slot, 4) || !aligned(topk_weights, 4))
    return EP_ERR_INVALID_ARG;
  if (grad_w != nullptr && (!aligned(y, 16) || !aligned(grad_w, 4))) return EP_ERR_INVALID_ARG;
  return from_hip(ep::launch_combine_backward(
      static_cast<const uint16_t*>(grad_out), static_cast<const uint16_t*>(y), slot, topk_weights,
      static_cast<int32_t>(num_tokens), hidden, top_k, static_cast<uint16_t*>(grad_y), grad_w,
      static_cast<hipStream_t>(stream)));
}

EP_API ep_status ep_cast_fp8_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return EP_ERR_INVALID_ARG;
  if (n >= kMaxCast) return EP_ERR_UNSUPPORTED;
  if (n == 0) return EP_OK;
  if (!in || !out || !aligned(in, 16) || !aligned(out, 16)) return EP_ERR_INVALID_ARG;
  return from_hip(ep::launch_cast_fp8(in, out, n, static_cast<hipStream_t>(stream)));
}
