// Combine: gather each token's K expert-output rows and reduce them to one
// BF16 row, weighted by topk_weights.
//
// [P5 "典型工作流程"]: combine reduces the expert outputs back to the
// source; [P1 "DeepEP 的常规内核和低延迟内核"]: the merge is in BF16.
// Arithmetic (not fixed by the pages): binary32, k ascending, each product
// rounded before it is added (__fmul_rn / __fadd_rn, so the compiler cannot
// fuse them), starting from +0.0, one BF16 round-to-nearest-even at the end.
// With no weights (w == nullptr) every weight is 1 (the product is exact):
// that is the backward of dispatch, which sums the gradients of a token's K
// copies ([P5 "典型工作流程"] lists backward helpers beside combine).
//
// gfx950 design: bound by HBM reads (K gathered rows per output row).  Work
// item = (token, 8 channels): the K row indices and weights are loaded
// first, then all K 16-byte gathers are issued before any arithmetic so that
// K loads per lane are in flight, then the ordered sum.  Large batches read
// the expert rows once and write the output once, so both use non-temporal
// (streaming) accesses: they neither allocate in nor evict from the caches,
// which on MI355X lifts a gather that otherwise competes with dirty-line
// write-back from ~3.5-5.0 TB/s to ~5.3-5.7 TB/s.  Small batches (under
// 64 MB of gathered rows, e.g. decode: 14.7 MB) use plain accesses, which
// hit rows still held in the caches (measured 3.1-3.3 against 3.8 us for
// 128 tokens, top-8, hidden 7168).  No LDS, no MFMA.

// Gathered bytes from which the streaming accesses are used.
constexpr size_t kStreamingBytes = size_t(64) << 20;

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;

// Adds the terms of k = k0 .. k0+KC-1 (those < K) to acc, in ascending k.
template <int KC, bool NT>
__device__ __forceinline__ void accumulate_chunk(const uint16_t* __restrict__ y, const int32_t* __restrict__ srow,
                                                 const float* __restrict__ wrow, int k0, int K, int32_t H,
                                                 uint32_t v, float (&acc)[8]) {
  int32_t r[KC];
  float wk[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const bool in = k0 + j < K;
    r[j] = in ? srow[k0 + j] : -1;
    wk[j] = in ? (wrow != nullptr ? wrow[k0 + j] : 1.0f) : 0.0f;  // no weights: unit weights
  }
  u32x4 d[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    d[j] = u32x4{0, 0, 0, 0};
    if (r[j] >= 0) {
      const u32x4* p = reinterpret_cast<const u32x4*>(y + static_cast<size_t>(r[j]) * H) + v;
      d[j] = NT ? __builtin_nontemporal_load(p) : *p;
    }
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (r[j] < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __fadd_rn(acc[2 * i], __fmul_rn(wk[j], bf16_lo(d[j][i])));
      acc[2 * i + 1] = __fadd_rn(acc[2 * i + 1], __fmul_rn(wk[j], bf16_hi(d[j][i])));
    }
  }
}

// UNIT: no weights (every weight 1), the backward of dispatch; a separate
// instantiation so profiles tell the two uses apart.  NT: streaming accesses.
template <int KT, bool UNIT, bool NT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                           const int32_t* __restrict__ slot,
                                                           const float* __restrict__ w, uint32_t n_items,
                                                           uint32_t vpt, int32_t H, int32_t Krt,
                                                           uint16_t* __restrict__ out) {
  const int K = KT > 0 ? KT : Krt;
  const uint32_t item = blockIdx.x * kThreads + threadIdx.x;
  if (item >= n_items) return;
  const uint32_t t = item / vpt;
  const uint32_t v = item - t * vpt;  // 8-channel vector within the token
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = UNIT ? nullptr : w + static_cast<size_t>(t) * K;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if (KT > 0) {
    accumulate_chunk<(KT > 0 ? KT : 1), NT>(y, srow, wrow, 0, K, H, v, acc);
  } else {
    for (int k0 = 0; k0 < K; k0 += 8) accumulate_chunk<8, NT>(y, srow, wrow, k0, K, H, v, acc);
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  u32x4* dst = reinterpret_cast<u32x4*>(out + static_cast<size_t>(t) * H) + v;
  if (NT)
    __builtin_nontemporal_store(o, dst);
  else
    *dst = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const int32_t* slot, const float* w, int32_t T, int32_t H,
                          int32_t K, uint16_t* out, hipStream_t stream) {
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t n_items = static_cast<uint32_t>(T) * vpt;
  if (n_items == 0) return hipSuccess;
  const dim3 grid((n_items + kThreads - 1) / kThreads), block(kThreads);
  const bool nt = static_cast<size_t>(T) * K * H * 2 >= kStreamingBytes;
#define EP_COMBINE_NT(KV, U, NTV) \
  hipLaunchKernelGGL((combine_kernel<KV, U, NTV>), grid, block, 0, stream, y, slot, w, n_items, vpt, H, K, out)
#define EP_COMBINE(KV)                                                     \
  if (w == nullptr) {                                                      \
    if (nt) EP_COMBINE_NT(KV, true, true); else EP_COMBINE_NT(KV, true, false);   \
  } else {                                                                 \
    if (nt) EP_COMBINE_NT(KV, false, true); else EP_COMBINE_NT(KV, false, false); \
  }
  switch (K) {
    case 1: { EP_COMBINE(1); } break;
    case 2: { EP_COMBINE(2); } break;
    case 4: { EP_COMBINE(4); } break;
    case 6: { EP_COMBINE(6); } break;
    case 8: { EP_COMBINE(8); } break;
    default: { EP_COMBINE(0); } break;
  }
#undef EP_COMBINE
#undef EP_COMBINE_NT
  return hipGetLastError();
}

}  // namespace ep
