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
//
// The per-item kernel issues its K gathers with no branch: a gather under
// a per-lane `if (row >= 0)` compiled, on gfx950, to the first two gathers,
// a wait for them, then the other six, i.e. two memory latencies per item
// instead of one.  Where a wavefront lies inside one token (H/8 a multiple
// of 64) the token's slots and weights are scalar loads.  At 128 tokens,
// top-8, hidden 7168 the kernel takes 2.84 against 3.12 us (GPU time of a
// replayed graph of back-to-back launches, one process, bit-equal).  The
// burst kernel keeps the branch: there the branch-free form measured the
// same or slower (84.8 against 84.5 us; the dispatch backward 84.8 against
// 82.7 us).
//
// Large batches (combine_burst_kernel): HBM moves a stream of reads alone
// faster than one with writes mixed in, so each 1024-lane workgroup (one
// per CU) owns ceil(T / CUs) consecutive tokens, keeps its finished output
// vectors in registers (at most kBurstItems per lane) and writes them all
// once the gathers of all its waves are done (a workgroup barrier): the
// writes of all CUs come at the end, in one burst, instead of among the
// reads.  At 4096 tokens x 7168, top-8, the barrier took the kernel from
// 84.2 to 81.5 us (the first wave of a workgroup had its reads in ~7 us
// before the last and started writing), 32768 tokens from 687 to 673 us.  A batch with more work items than
// the workgroups can hold is split into equal slices of tokens, one launch
// each (T <= 4096 at hidden 7168 is one launch).

// Gathered bytes from which the streaming accesses are used.
constexpr size_t kStreamingBytes = size_t(64) << 20;

#include "burst_plan.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kBurstThreads = 1024;
constexpr int kBurstItems = 14;  // output vectors held per lane (4 VGPRs each)

// Adds the terms of k = k0 .. k0+KC-1 (those < K) to acc, in ascending k.
// UNIT: every weight 1 (wrow unused).  UNCOND: no gather under a branch.
template <int KC, bool UNIT, bool NT, bool UNCOND = false>
__device__ __forceinline__ void accumulate_chunk(const uint16_t* __restrict__ y, const int32_t* __restrict__ srow,
                                                 const float* __restrict__ wrow, int k0, int K, int32_t H,
                                                 uint32_t v, float (&acc)[8]) {
  int32_t r[KC];
  float wk[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const bool in = k0 + j < K;
    r[j] = in ? srow[k0 + j] : -1;
    wk[j] = UNIT ? 1.0f : (in ? wrow[k0 + j] : 0.0f);
  }
  u32x4 d[KC];
  if constexpr (UNCOND) {
    // every gather issued, none under a branch: a masked entry reads row 0
    // (every y has one) and its term is replaced by +0.0; acc starts at +0.0
    // and a sum of binary32 terms that is exactly zero is +0.0, so acc is
    // never -0.0 and acc + 0.0 == acc: the result is that of skipping it
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const u32x4* p = reinterpret_cast<const u32x4*>(y + static_cast<size_t>(r[j] < 0 ? 0 : r[j]) * H) + v;
      d[j] = NT ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bool m = r[j] < 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __fmul_rn(wk[j], bf16_lo(d[j][i])), hi = __fmul_rn(wk[j], bf16_hi(d[j][i]));
        acc[2 * i] = __fadd_rn(acc[2 * i], m ? 0.0f : lo);
        acc[2 * i + 1] = __fadd_rn(acc[2 * i + 1], m ? 0.0f : hi);
      }
    }
    return;
  }
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
template <int KT, bool UNIT, bool NT, bool WU = false>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                           const int32_t* __restrict__ slot,
                                                           const float* __restrict__ w, uint32_t n_items,
                                                           uint32_t vpt, int32_t H, int32_t Krt,
                                                           uint16_t* __restrict__ out) {
  const int K = KT > 0 ? KT : Krt;
  const uint32_t item = blockIdx.x * kThreads + threadIdx.x;
  if (item >= n_items) return;
  // WU: every wavefront lies inside one token (vpt a multiple of 64), so the
  // token index is wave-uniform and its slots and weights are scalar loads
  const uint32_t t = WU ? __builtin_amdgcn_readfirstlane(item / vpt) : item / vpt;
  const uint32_t v = item - t * vpt;  // 8-channel vector within the token
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = UNIT ? nullptr : w + static_cast<size_t>(t) * K;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if (KT > 0) {
    accumulate_chunk<(KT > 0 ? KT : 1), UNIT, NT, true>(y, srow, wrow, 0, K, H, v, acc);
  } else {
    for (int k0 = 0; k0 < K; k0 += 8) accumulate_chunk<8, UNIT, NT, true>(y, srow, wrow, k0, K, H, v, acc);
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

// Workgroup b: tokens b*tpb .. b*tpb+tpb-1, whose work items i*kBurstThreads
// + tid, i < kBurstItems, this lane sums as combine_kernel does; the output
// vectors are held until every item of the lane is summed, then written.
template <int KT, bool UNIT>
__global__ __launch_bounds__(kBurstThreads) void combine_burst_kernel(const uint16_t* __restrict__ y,
                                                                      const int32_t* __restrict__ slot,
                                                                      const float* __restrict__ w, int32_t T,
                                                                      int32_t H, int32_t Krt, int32_t tpb,
                                                                      uint16_t* __restrict__ out) {
  const int K = KT > 0 ? KT : Krt;
  const int tok0 = blockIdx.x * tpb;
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t nitems = static_cast<uint32_t>(min(T - tok0, tpb)) * vpt;
  u32x4 o[kBurstItems];
#pragma unroll
  for (int i = 0; i < kBurstItems; ++i) {
    const uint32_t item = static_cast<uint32_t>(i * kBurstThreads) + threadIdx.x;
    if (item < nitems) {
      const uint32_t tl = item / vpt, v = item - tl * vpt;
      const int32_t* srow = slot + static_cast<size_t>(tok0 + tl) * K;
      const float* wrow = UNIT ? nullptr : w + static_cast<size_t>(tok0 + tl) * K;
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
      if (KT > 0) {
        accumulate_chunk<(KT > 0 ? KT : 1), UNIT, true>(y, srow, wrow, 0, K, H, v, acc);
      } else {
        for (int k0 = 0; k0 < K; k0 += 8) accumulate_chunk<8, UNIT, true>(y, srow, wrow, k0, K, H, v, acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) o[i][q] = f32_to_bf16_rne(acc[2 * q]) | (f32_to_bf16_rne(acc[2 * q + 1]) << 16);
    }
  }
  // no wave writes before every wave of the workgroup has its reads in:
  // the first waves finish their gathers several us before the last, and
  // their writes would otherwise mix into the CU's remaining reads
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBurstItems; ++i) {
    const uint32_t item = static_cast<uint32_t>(i * kBurstThreads) + threadIdx.x;
    if (item < nitems) {
      const uint32_t tl = item / vpt, v = item - tl * vpt;
      __builtin_nontemporal_store(o[i], reinterpret_cast<u32x4*>(out + static_cast<size_t>(tok0 + tl) * H) + v);
    }
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const int32_t* slot, const float* w, int32_t T, int32_t H,
                          int32_t K, uint16_t* out, hipStream_t stream) {
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t n_items = static_cast<uint32_t>(T) * vpt;
  if (n_items == 0) return hipSuccess;
  const dim3 grid((n_items + kThreads - 1) / kThreads), block(kThreads);
  const bool nt = static_cast<size_t>(T) * K * H * 2 >= kStreamingBytes;
  // burst: large batches, one workgroup per CU, in equal token slices of at
  // most one held round each
  const int cus = nt ? device_cu_count() : 0;
  const BurstPlan plan = burst_plan(T, vpt, kBurstItems, kBurstThreads, cus, 0, 0);
  if (plan.launches > 0) {
    for (int t0 = 0; t0 < T; t0 += plan.slice) {
      const int Ts = min(plan.slice, T - t0);
      const int tpb = burst_tpb(Ts, cus);
      const dim3 bgrid((Ts + tpb - 1) / tpb), bblock(kBurstThreads);
      const int32_t* sl = slot + static_cast<size_t>(t0) * K;
      const float* ws = w != nullptr ? w + static_cast<size_t>(t0) * K : nullptr;
      uint16_t* os = out + static_cast<size_t>(t0) * H;
#define EP_COMBINE_BURST(KV)                                                                                    \
  if (ws == nullptr)                                                                                            \
    hipLaunchKernelGGL((combine_burst_kernel<KV, true>), bgrid, bblock, 0, stream, y, sl, ws, Ts, H, K, tpb, os); \
  else                                                                                                          \
    hipLaunchKernelGGL((combine_burst_kernel<KV, false>), bgrid, bblock, 0, stream, y, sl, ws, Ts, H, K, tpb, os)
      switch (K) {
        case 1: { EP_COMBINE_BURST(1); } break;
        case 2: { EP_COMBINE_BURST(2); } break;
        case 4: { EP_COMBINE_BURST(4); } break;
        case 6: { EP_COMBINE_BURST(6); } break;
        case 8: { EP_COMBINE_BURST(8); } break;
        default: { EP_COMBINE_BURST(0); } break;
      }
#undef EP_COMBINE_BURST
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
#define EP_COMBINE_NT(KV, U, NTV)                                                                             \
  if (vpt % kWave == 0)                                                                                       \
    hipLaunchKernelGGL((combine_kernel<KV, U, NTV, true>), grid, block, 0, stream, y, slot, w, n_items, vpt, H, \
                       K, out);                                                                               \
  else                                                                                                        \
    hipLaunchKernelGGL((combine_kernel<KV, U, NTV, false>), grid, block, 0, stream, y, slot, w, n_items, vpt, H, \
                       K, out)
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
