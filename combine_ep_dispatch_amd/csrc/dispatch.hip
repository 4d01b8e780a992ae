// Dispatch: copy every token into its K expert-major receive rows, either
// quantised to OCP E4M3FN with one binary32 scale per 128 channels, or as
// the unchanged BF16 bits.
//
// [P1 "DeepEP 的常规内核和低延迟内核"]: tokens are sent to their experts in
// FP8.  Scale rule (not given by the pages): s = RN32(amax / 448) per
// 128-channel group (1 for an all-zero group, floored at 2^-126), code =
// E4M3_RNE(RN32(x / s)).
//
// gfx950 design: pure data movement, bound by HBM writes (K copies of every
// token).  The token is the unit of work, never the expert, so skewed
// routing cannot unbalance the CUs.  Work item = (token, 16 channels) for FP8
// (two 16-byte loads, one 16-byte store per copy) or (token, 8 channels) for
// BF16 (one 16-byte load, K 16-byte stores).  Eight consecutive lanes hold
// one 128-channel group, so the group max is three DPP steps inside the
// wavefront; the division is IEEE correctly rounded (no reciprocal
// shortcut), and the conversion is gfx950's OCP FP8 convert.  The token is
// read once, with non-temporal loads (about 10% faster at 4096 tokens), or
// with plain loads when the batch is small enough to be cache-resident
// (under 16 MB of tokens, e.g. decode); the receive rows are written with
// plain stores: for these scattered 1 KB row segments (one wave's 64
// 16-byte stores) they measured 6.1 TB/s on MI355X, non-temporal ones
// 2.3 TB/s.
// Not ALU-bound: replacing the division by a reciprocal multiply is not
// measurably faster.  No LDS, no MFMA.

#include "burst_plan.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;

// Receive rows (and weights) of entries k0 .. k0+KC-1 of one token, loaded
// together before any store so their latencies overlap.  The row loads
// have no per-lane condition, and the weights are loaded by every lane of
// a wave that needs them (load_w is wave-uniform; wrow is then valid): a
// load under a per-lane branch makes the compiler wait for each load
// before issuing the next.
template <int KC>
__device__ __forceinline__ void load_rows(const int32_t* __restrict__ srow, const float* __restrict__ wrow,
                                          int k0, int K, bool load_w, int32_t (&r)[KC], float (&wk)[KC]) {
#pragma unroll
  for (int j = 0; j < KC; ++j) r[j] = k0 + j < K ? srow[k0 + j] : -1;
#pragma unroll
  for (int j = 0; j < KC; ++j) wk[j] = 0.0f;
  if (load_w) {
#pragma unroll
    for (int j = 0; j < KC; ++j) wk[j] = k0 + j < K ? wrow[k0 + j] : 0.0f;
  }
}

// WS: every wavefront lies inside one token (H/16 a multiple of 64) and
// recv_scale takes 16-byte stores, so the scales go out 32 bytes per row
// (store_wave_scales); otherwise one lane per group stores its scale.
template <int KT, bool NT, bool WS>
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const uint16_t* __restrict__ x, uint32_t n_items, uint32_t vpt, int32_t H, int32_t Krt,
    const int32_t* __restrict__ slot, const float* __restrict__ w, uint8_t* __restrict__ recv,
    float* __restrict__ recv_scale, float* __restrict__ recv_weight) {
  constexpr int KC = KT > 0 ? KT : 8;  // receive rows handled per pass
  const int K = KT > 0 ? KT : Krt;
  const uint32_t item = blockIdx.x * kThreads + threadIdx.x;
  const bool active = item < n_items;
  const uint32_t t = active ? item / vpt : 0;
  const uint32_t v = item - t * vpt;  // 16-channel vector within the token
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = w != nullptr ? w + static_cast<size_t>(t) * K : nullptr;
  const bool want_w = recv_weight != nullptr && v == 0;

  // the token's loads first, then the receive rows: all are in flight
  // before anything waits for one of them
  u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
  if (active) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * H) + 2 * v;
    a = load_token<NT>(src);
    b = load_token<NT>(src + 1);
  }
  int32_t r[KC];
  float wk[KC];
  if (active) load_rows<KC>(srow, wrow, 0, K, recv_weight != nullptr, r, wk);
  const int lane = threadIdx.x & (kWave - 1);
  int32_t rj = -1;  // WS: this lane's row for the scale stores
  if (WS && active && lane < KC && lane < K) rj = srow[lane];
  float s;
  const u32x4 q = quantize16_e4m3(a, b, s);

  if (!active) return;  // with WS whole wavefronts only
  const uint32_t G = static_cast<uint32_t>(H) / kGroup;
  const bool lead = (v & 7) == 0;  // one lane per group writes the scale
  for (int k0 = 0;;) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (r[j] < 0) continue;
      reinterpret_cast<u32x4*>(recv + static_cast<size_t>(r[j]) * H)[v] = q;
      if (!WS && lead) {
        float* ps = recv_scale + static_cast<size_t>(r[j]) * G + (v >> 3);
        if (NT) __builtin_nontemporal_store(s, ps); else *ps = s;
      }
      if (want_w) recv_weight[r[j]] = wk[j];
    }
    if (WS) store_wave_scales<NT>(rj, s, v, G, recv_scale);
    k0 += KC;
    if (k0 >= K) break;
    load_rows<KC>(srow, wrow, k0, K, recv_weight != nullptr, r, wk);
    if (WS) rj = lane < KC && k0 + lane < K ? srow[k0 + lane] : -1;
  }
}

template <int KT, bool NT>
__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const uint16_t* __restrict__ x, uint32_t n_items, uint32_t vpt, int32_t H, int32_t Krt,
    const int32_t* __restrict__ slot, const float* __restrict__ w, uint16_t* __restrict__ recv,
    float* __restrict__ recv_weight) {
  constexpr int KC = KT > 0 ? KT : 8;
  const int K = KT > 0 ? KT : Krt;
  const uint32_t item = blockIdx.x * kThreads + threadIdx.x;
  if (item >= n_items) return;
  const uint32_t t = item / vpt;
  const uint32_t v = item - t * vpt;  // 8-channel vector within the token
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = w != nullptr ? w + static_cast<size_t>(t) * K : nullptr;
  const bool want_w = recv_weight != nullptr && v == 0;
  const u32x4 d = load_token<NT>(reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * H) + v);
  int32_t r[KC];
  float wk[KC];
  load_rows<KC>(srow, wrow, 0, K, recv_weight != nullptr, r, wk);
  for (int k0 = 0;;) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (r[j] < 0) continue;
      reinterpret_cast<u32x4*>(recv + static_cast<size_t>(r[j]) * H)[v] = d;
      if (want_w) recv_weight[r[j]] = wk[j];
    }
    k0 += KC;
    if (k0 >= K) break;
    load_rows<KC>(srow, wrow, k0, K, recv_weight != nullptr, r, wk);
  }
}

// Burst fan-out of BF16 token rows (the BF16 dispatch, and the combine
// backward's row gradients): HBM writes faster when no reads are mixed in,
// so each 1024-lane workgroup (one per CU) owns tpb consecutive tokens,
// loads all its work items (token, 8 channels) first, up to kFanItems per
// lane, with the tokens' K receive rows (and weights) staged in LDS, and
// then writes the K copies.  WEIGHTED: copy k is BF16_RNE(RN32(w[t,k] *
// x[t,c])) per channel; else the bits unchanged, with recv_weight[r] =
// w[t,k] when recv_weight is given.
constexpr int kFanThreads = 1024;
constexpr int kFanItems = 14;  // token vectors held per lane (4 VGPRs each)

template <bool WEIGHTED, bool NT>
__global__ __launch_bounds__(kFanThreads) void fanout_burst_bf16(const uint16_t* __restrict__ x,
                                                                 const int32_t* __restrict__ slot,
                                                                 const float* __restrict__ w, int32_t T, int32_t H,
                                                                 int32_t K, int32_t tpb, uint16_t* __restrict__ out,
                                                                 float* __restrict__ recv_weight) {
  extern __shared__ int32_t fan_lds[];  // rows [tpb*K], then weights [tpb*K]
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * tpb;
  const int ntok = min(T - tok0, tpb);
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t nitems = static_cast<uint32_t>(ntok) * vpt;
  const int nit = static_cast<int>((nitems + kFanThreads - 1) / kFanThreads);  // workgroup-uniform
  u32x4 d[kFanItems];
  static_for<0, kFanItems>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (i >= nit) return;
    const uint32_t item = min(static_cast<uint32_t>(i * kFanThreads + tid), nitems - 1);
    const uint32_t tl = item / vpt;
    d[i] = load_token<NT>(reinterpret_cast<const u32x4*>(x + static_cast<size_t>(tok0 + tl) * H) + (item - tl * vpt));
  });
  const bool need_w = WEIGHTED || recv_weight != nullptr;
  int32_t* rows = fan_lds;
  float* wts = reinterpret_cast<float*>(fan_lds + tpb * K);
  for (int e = tid; e < ntok * K; e += kFanThreads) {
    rows[e] = slot[static_cast<size_t>(tok0) * K + e];
    if (need_w) wts[e] = w[static_cast<size_t>(tok0) * K + e];
  }
  __syncthreads();
  static_for<0, kFanItems>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const uint32_t item = static_cast<uint32_t>(i * kFanThreads + tid);
    if (i >= nit || item >= nitems) return;
    const uint32_t tl = item / vpt, v = item - tl * vpt;
    const int32_t* tr = rows + tl * K;
    const float* tw = wts + tl * K;
    for (int k = 0; k < K; ++k) {
      const int r = tr[k];
      if (r < 0) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * H) + v;
      if constexpr (WEIGHTED) {
        const float wk = tw[k];
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = f32_to_bf16_rne(__fmul_rn(wk, bf16_lo(d[i][q]))) | (f32_to_bf16_rne(__fmul_rn(wk, bf16_hi(d[i][q]))) << 16);
        *dst = o;
      } else {
        *dst = d[i];
        if (recv_weight != nullptr && v == 0) recv_weight[r] = tw[k];
      }
    }
  });
}

__global__ __launch_bounds__(kThreads) void cast_fp8_kernel(const float* __restrict__ in,
                                                            uint8_t* __restrict__ out, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *reinterpret_cast<const float4*>(in + i);
    *reinterpret_cast<uint32_t*>(out + i) = f32x4_to_e4m3(v.x, v.y, v.z, v.w);
  } else if (i < n) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; i + j < n; ++j) v[j] = in[i + j];
    const uint32_t c = f32x4_to_e4m3(v[0], v[1], v[2], v[3]);
    for (int j = 0; i + j < n; ++j) out[i + j] = static_cast<uint8_t>(c >> (8 * j));
  }
}

}  // namespace

hipError_t launch_dispatch_fp8(const uint16_t* x, int32_t T, int32_t H, int32_t K, const int32_t* slot,
                               const float* w, uint8_t* recv, float* recv_scale, float* recv_weight,
                               hipStream_t stream) {
  const uint32_t vpt = static_cast<uint32_t>(H) / 16;
  const uint32_t n_items = static_cast<uint32_t>(T) * vpt;
  if (n_items == 0) return hipSuccess;
  const dim3 grid((n_items + kThreads - 1) / kThreads), block(kThreads);
  const bool nt = static_cast<size_t>(T) * H * 2 >= kStreamingTokenBytes;
  // wavefronts inside one token (vpt a multiple of 64: H a multiple of 1024)
  // and 16-byte pieces of the scale rows (G a multiple of 4, aligned base)
  const bool ws = vpt % kWave == 0 && (H / kGroup) % 4 == 0 && (reinterpret_cast<uintptr_t>(recv_scale) & 15) == 0;
#define EP_DISPATCH_FP8_V(KV, NTV, WSV)                                                                           \
  hipLaunchKernelGGL((dispatch_fp8_kernel<KV, NTV, WSV>), grid, block, 0, stream, x, n_items, vpt, H, K, slot, w, \
                     recv, recv_scale, recv_weight)
#define EP_DISPATCH_FP8(KV)                                              \
  if (nt) {                                                              \
    if (ws) EP_DISPATCH_FP8_V(KV, true, true); else EP_DISPATCH_FP8_V(KV, true, false);   \
  } else {                                                               \
    if (ws) EP_DISPATCH_FP8_V(KV, false, true); else EP_DISPATCH_FP8_V(KV, false, false); \
  }
  switch (K) {
    case 1: { EP_DISPATCH_FP8(1); } break;
    case 2: { EP_DISPATCH_FP8(2); } break;
    case 4: { EP_DISPATCH_FP8(4); } break;
    case 6: { EP_DISPATCH_FP8(6); } break;
    case 8: { EP_DISPATCH_FP8(8); } break;
    default: { EP_DISPATCH_FP8(0); } break;
  }
#undef EP_DISPATCH_FP8
#undef EP_DISPATCH_FP8_V
  return hipGetLastError();
}

bool launch_fanout_burst_bf16(const uint16_t* x, const int32_t* slot, const float* w, int32_t T, int32_t H,
                              int32_t K, bool weighted, uint16_t* out, float* recv_weight, hipStream_t stream,
                              hipError_t* err) {
  // tokens of 16 MB and more (read once, non-temporal), one workgroup per
  // CU, in equal token slices of at most kFanItems vectors per lane each
  // (each token stages its K rows and weights in LDS: 8K bytes)
  if (static_cast<size_t>(T) * H * 2 < kStreamingTokenBytes) return false;
  const int cus = device_cu_count();
  const size_t lds_per_token = static_cast<size_t>(K) * 8;
  const BurstPlan plan = burst_plan(T, H / 8, kFanItems, kFanThreads, cus, lds_per_token, kLdsLimit);
  if (plan.launches == 0) return false;
  for (int t0 = 0; t0 < T; t0 += plan.slice) {
    const int Ts = min(plan.slice, T - t0);
    const int tpb = burst_tpb(Ts, cus);
    const dim3 grid((Ts + tpb - 1) / tpb), block(kFanThreads);
    const size_t lds = static_cast<size_t>(tpb) * lds_per_token;
    const int32_t* sl = slot + static_cast<size_t>(t0) * K;
    const float* ws = w != nullptr ? w + static_cast<size_t>(t0) * K : nullptr;
    const uint16_t* xs = x + static_cast<size_t>(t0) * H;
    if (weighted)
      hipLaunchKernelGGL((fanout_burst_bf16<true, true>), grid, block, lds, stream, xs, sl, ws, Ts, H, K, tpb, out,
                         nullptr);
    else
      hipLaunchKernelGGL((fanout_burst_bf16<false, true>), grid, block, lds, stream, xs, sl, ws, Ts, H, K, tpb, out,
                         recv_weight);
    *err = hipGetLastError();
    if (*err != hipSuccess) return true;
  }
  return true;
}

hipError_t launch_dispatch_bf16(const uint16_t* x, int32_t T, int32_t H, int32_t K, const int32_t* slot,
                                const float* w, uint16_t* recv, float* recv_weight, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (launch_fanout_burst_bf16(x, slot, w, T, H, K, false, recv, recv_weight, stream, &e)) return e;
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t n_items = static_cast<uint32_t>(T) * vpt;
  if (n_items == 0) return hipSuccess;
  const dim3 grid((n_items + kThreads - 1) / kThreads), block(kThreads);
  const bool nt = static_cast<size_t>(T) * H * 2 >= kStreamingTokenBytes;
#define EP_DISPATCH_BF16(KV)                                                                                 \
  if (nt)                                                                                                    \
    hipLaunchKernelGGL((dispatch_bf16_kernel<KV, true>), grid, block, 0, stream, x, n_items, vpt, H, K, slot, w, \
                       recv, recv_weight);                                                                   \
  else                                                                                                       \
    hipLaunchKernelGGL((dispatch_bf16_kernel<KV, false>), grid, block, 0, stream, x, n_items, vpt, H, K, slot, w, \
                       recv, recv_weight)
  switch (K) {
    case 1: { EP_DISPATCH_BF16(1); } break;
    case 2: { EP_DISPATCH_BF16(2); } break;
    case 4: { EP_DISPATCH_BF16(4); } break;
    case 6: { EP_DISPATCH_BF16(6); } break;
    case 8: { EP_DISPATCH_BF16(8); } break;
    default: { EP_DISPATCH_BF16(0); } break;
  }
#undef EP_DISPATCH_BF16
  return hipGetLastError();
}

hipError_t launch_cast_fp8(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const dim3 grid(static_cast<uint32_t>((threads + kThreads - 1) / kThreads)), block(kThreads);
  hipLaunchKernelGGL(cast_fp8_kernel, grid, block, 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace ep
