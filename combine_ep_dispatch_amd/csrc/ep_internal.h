// Host-side launchers for the kernels (internal; the C ABI in ep_api.hip
// validates arguments and then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Layout: chooses the single-workgroup path or the two-kernel multi-block
// path from the shape.
size_t layout_workspace_bytes(int64_t rows, int32_t num_experts);
// capacity == 0: packed layout (counts, offsets, slot, src[T*K]);
// capacity  > 0: padded layout (counts clamped, offsets unused, src[E*capacity]).
// Idx: int32_t or int64_t expert ids.
template <typename Idx>
hipError_t launch_layout(const Idx* topk_idx, int32_t rows, int32_t top_k, int32_t num_experts, int32_t capacity,
                         int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src, void* workspace,
                         hipStream_t stream);

hipError_t launch_dispatch_fp8(const uint16_t* x, int32_t num_tokens, int32_t hidden, int32_t top_k,
                               const int32_t* slot, const float* topk_weights, uint8_t* recv,
                               float* recv_scale, float* recv_weight, hipStream_t stream);

hipError_t launch_dispatch_bf16(const uint16_t* x, int32_t num_tokens, int32_t hidden, int32_t top_k,
                                const int32_t* slot, const float* topk_weights, uint16_t* recv,
                                float* recv_weight, hipStream_t stream);

// The burst fan-out of BF16 token rows (from 16 MB of tokens): out[slot[t,k]]
// = x[t] (weighted: BF16_RNE(RN32(w[t,k] * x[t])) per channel); returns false,
// launching nothing, below its size or where the device's CU count is unknown.
bool launch_fanout_burst_bf16(const uint16_t* x, const int32_t* slot, const float* w, int32_t T, int32_t H,
                              int32_t K, bool weighted, uint16_t* out, float* recv_weight, hipStream_t stream,
                              hipError_t* err);

// topk_weights == nullptr: unit weights (the backward of dispatch)
hipError_t launch_combine(const uint16_t* y, const int32_t* slot, const float* topk_weights,
                          int32_t num_tokens, int32_t hidden, int32_t top_k, uint16_t* out,
                          hipStream_t stream);

// grad_w may be null (then y is not read)
hipError_t launch_combine_backward(const uint16_t* grad_out, const uint16_t* y, const int32_t* slot,
                                   const float* w, int32_t num_tokens, int32_t hidden, int32_t top_k,
                                   uint16_t* grad_y, float* grad_w, hipStream_t stream);

// Layout and dispatch together (ep_layout_dispatch): the decode kernel when
// num_tokens * top_k <= kFusedMaxEntries; up to kOneLaunchMaxEntries the
// chunked kernel where its shape limits allow; else launch_layout followed by
// the dispatch kernel (then `workspace` must hold layout_workspace_bytes).
constexpr int kFusedMaxEntries = 3072;
constexpr int kOneLaunchMaxEntries = 65536;  // the one-launch layout (no workspace)
template <typename Idx>
hipError_t launch_layout_dispatch(const Idx* topk_idx, const uint16_t* x, const float* topk_weights,
                                  int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                  int32_t capacity, bool fp8, int32_t* counts, int32_t* offsets, int32_t* slot,
                                  int32_t* src, void* recv, float* recv_scale, float* recv_weight,
                                  void* workspace, hipStream_t stream);

// The chunked layout + dispatch kernel: returns false, launching nothing,
// when the shape is outside its limits; else launches and sets *err.
template <typename Idx>
bool launch_layout_dispatch_chunked(const Idx* topk_idx, const uint16_t* x, const float* topk_weights,
                                    int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                    int32_t capacity, bool fp8, int32_t* counts, int32_t* offsets, int32_t* slot,
                                    int32_t* src, void* recv, float* recv_scale, float* recv_weight,
                                    hipStream_t stream, hipError_t* err);

// Compute units of the current device (read once per device; 0 if the
// runtime cannot tell).  Kernels that size their grid at one workgroup per
// CU take it from here, so a partitioned GPU gets a grid that fits it.
int device_cu_count();

// Dispatch reads the tokens with non-temporal loads from this many bytes of
// tokens on (they are read once); smaller batches are usually still cached.
constexpr size_t kStreamingTokenBytes = size_t(16) << 20;

hipError_t launch_cast_fp8(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace ep
