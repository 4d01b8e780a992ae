// Backward of combine: gradients w.r.t. the expert outputs and the routing
// weights ([P5 "典型工作流程"] lists backward helpers beside combine; the
// pages give no arithmetic for them).
//
// combine computes out[t] = sum_k w[t,k] * y[slot[t,k]], so
//   grad_y[slot[t,k], c] = BF16_RNE(RN32(w[t,k] * grad_out[t,c]))
//   grad_w[t,k]          = sum_c grad_out[t,c] * y[slot[t,k], c]
// The dot product has a fixed order, so results are reproducible run to
// run: the 8 products of each 8-channel vector (exact: BF16 x BF16 fits
// binary32) are added in channel order into +0.0, then the H/8 vector sums
// are added as a binary tree of depth ceil(log2(H/8)): 6 levels across a
// wavefront (lanes past the last vector add +0.0, which is exact), then a
// tree over the waves.  Each product thus passes through at most
// 7 + ceil(log2(H/8)) rounded additions, which bounds the distance to the
// exact dot product by that many units of 2^-24 times sum |grad_out * y|
// (recursive summation error).
//
// gfx950 design: two HBM-bound kernels, which on MI355X measured ~13%
// faster than one kernel doing both (the reads then run without the
// scattered row writes in the same waves):
//  * `grad_rows_kernel`: the weighted fan-out, shaped like dispatch (work
//    item = (token, 8 channels), the K row indices first, one non-temporal
//    load of grad_out, K plain 16-byte stores); per token 2H + 8K bytes in,
//    2KH out.
//  * `grad_weights_kernel`: one workgroup per token, one lane per 8
//    channels (H <= 8192), reads grad_out and the K expert-row vectors
//    (non-temporal; all issued before any wait, none under a per-lane
//    condition: such a load is waited for before the next ones are issued)
//    and forms K vector sums (FMA: the products are exact, so this is the
//    add of the product).  For 8 sums at a time a wave reduces them
//    together by halving exchanges (wave_sum8: 34 operations against 8
//    separate trees, the two cross-row steps on the gfx950 lane swaps
//    instead of LDS permutes); lanes 0, 2, .., 14 of each wave park the
//    sums in LDS and K lanes finish the tree over the waves.  Measured at
//    4096 tokens x 7168, top-8: ep_combine_backward 181.8 against 184.7 us
//    (one workgroup per token reads these bytes alone in 77.4 us).
//    Per token 2H + 2KH + 4K bytes in, 4K out.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxWaves = 16;  // workgroups of up to 1024 lanes
constexpr int kMaxK = 32;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x + (the same register of lane i^16) resp. (lane i^32): the gfx950 lane
// swaps exchange half the rows, and both lanes of a pair add the same two
// values (a + b == b + a exactly).
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The 8 values p[0..7] of every lane summed over the 64 lanes, as 8 binary
// trees of depth 6, by halving exchanges (each lane sends the half its
// partner keeps): row_mirror pairs lane i with 15-i (lanes i%16 < 8 keep
// p[0..3]), row_half_mirror pairs i with 7-i (i%8 < 4 keep the first two),
// quad_perm [3,2,1,0] pairs i with 3-i (i%4 < 2 keep the first); then
// lanes i, i^1 hold the same partial and are added, and so are lanes i^16
// and i^32.  Lane i ends with the total of p[(i%16) >> 1].  34 operations
// instead of 8 separate wave trees.
__device__ __forceinline__ float wave_sum8(const float (&p)[8]) {
  const int i = threadIdx.x;
  const bool f1 = (i & 15) < 8, f2 = (i & 7) < 4, f3 = (i & 3) < 2;
  float q[4], r[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float send = f1 ? p[m + 4] : p[m], keep = f1 ? p[m] : p[m + 4];
    q[m] = __fadd_rn(keep, dpp_f32<0x140>(send));  // row_mirror
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float send = f2 ? q[m + 2] : q[m], keep = f2 ? q[m] : q[m + 2];
    r[m] = __fadd_rn(keep, dpp_f32<0x141>(send));  // row_half_mirror
  }
  const float send = f3 ? r[1] : r[0], keep = f3 ? r[0] : r[1];
  float u = __fadd_rn(keep, dpp_f32<0x1B>(send));  // quad_perm [3,2,1,0]
  u = __fadd_rn(u, dpp_f32<0xB1>(u));              // quad_perm [1,0,3,2]: lane i^1
  return add_xor32(add_xor16(u));
}

// Sum over the 64 lanes as a complete binary tree of adjacent lanes; every
// lane returns the total.
__device__ __forceinline__ float wave_tree_sum(float x) {
  x = __fadd_rn(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]: lane i^1
  x = __fadd_rn(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]: lane i^2
  x = __fadd_rn(x, dpp_f32<0x141>(x));  // row_half_mirror: 4-lane blocks pair up
  x = __fadd_rn(x, dpp_f32<0x140>(x));  // row_mirror: 8-lane blocks pair up
  x = __fadd_rn(x, __shfl_xor(x, 16, kWave));
  x = __fadd_rn(x, __shfl_xor(x, 32, kWave));
  return x;
}

template <int KT>
__global__ __launch_bounds__(kRowThreads) void grad_rows_kernel(const uint16_t* __restrict__ grad_out,
                                                                const int32_t* __restrict__ slot,
                                                                const float* __restrict__ w, uint32_t n_items,
                                                                uint32_t vpt, int32_t H, int32_t Krt,
                                                                uint16_t* __restrict__ grad_y) {
  constexpr int KC = KT > 0 ? KT : 8;
  const int K = KT > 0 ? KT : Krt;
  const uint32_t item = blockIdx.x * kRowThreads + threadIdx.x;
  if (item >= n_items) return;
  const uint32_t t = item / vpt;
  const uint32_t v = item - t * vpt;  // 8-channel vector within the token
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = w + static_cast<size_t>(t) * K;
  int32_t r[KC];
  float wk[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    r[j] = j < K ? srow[j] : -1;
    wk[j] = j < K ? wrow[j] : 0.0f;
  }
  const u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(grad_out + static_cast<size_t>(t) * H) + v);
  float g[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g[2 * i] = bf16_lo(gv[i]);
    g[2 * i + 1] = bf16_hi(gv[i]);
  }
  for (int k0 = 0;;) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (r[j] < 0) continue;
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_rne(__fmul_rn(wk[j], g[2 * i])) | (f32_to_bf16_rne(__fmul_rn(wk[j], g[2 * i + 1])) << 16);
      reinterpret_cast<u32x4*>(grad_y + static_cast<size_t>(r[j]) * H)[v] = o;
    }
    k0 += KC;
    if (k0 >= K) break;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      r[j] = k0 + j < K ? srow[k0 + j] : -1;
      wk[j] = k0 + j < K ? wrow[k0 + j] : 0.0f;
    }
  }
}

template <int KC>
__device__ __forceinline__ void weights_chunk(const uint16_t* __restrict__ y, const int32_t* __restrict__ srow,
                                              int k0, int K, int32_t H, uint32_t v, bool act, const float (&g)[8],
                                              float* wpart) {
  int32_t r[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) r[j] = k0 + j < K ? srow[k0 + j] : -1;
  u32x4 d[KC];
  if constexpr (KC == 8) {
    // every gather issued, none under a branch: a masked entry reads row 0
    // (its sum is discarded) and a lane past the last vector reads vector 0
    // (its sums are replaced by +0.0)
    const uint32_t vv = act ? v : 0u;
#pragma unroll
    for (int j = 0; j < KC; ++j)
      d[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + static_cast<size_t>(r[j] < 0 ? 0 : r[j]) * H) + vv);
    float part[8];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      // the products are exact (BF16 x BF16), so the FMA adds them as an
      // add of the rounded product would
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a = __builtin_fmaf(g[2 * i], bf16_lo(d[j][i]), a);
        a = __builtin_fmaf(g[2 * i + 1], bf16_hi(d[j][i]), a);
      }
      part[j] = act ? a : 0.0f;
    }
    const float tot = wave_sum8(part);
    const int lane = threadIdx.x & (kWave - 1);
    if (lane < 16 && (lane & 1) == 0 && k0 + (lane >> 1) < K)
      wpart[(threadIdx.x / kWave) * kMaxK + k0 + (lane >> 1)] = tot;
    return;
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    d[j] = u32x4{0, 0, 0, 0};
    if (act && r[j] >= 0)
      d[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + static_cast<size_t>(r[j]) * H) + v);
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (k0 + j >= K) break;  // wave-uniform
    float part = -0.0f;      // lanes past the last vector are tree padding
    if (act) {
      part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = __fadd_rn(part, __fmul_rn(g[2 * i], bf16_lo(d[j][i])));
        part = __fadd_rn(part, __fmul_rn(g[2 * i + 1], bf16_hi(d[j][i])));
      }
    }
    part = wave_tree_sum(part);
    if ((threadIdx.x & (kWave - 1)) == 0) wpart[(threadIdx.x / kWave) * kMaxK + k0 + j] = part;
  }
}

template <int KT>
__global__ __launch_bounds__(1024) void grad_weights_kernel(const uint16_t* __restrict__ grad_out,
                                                            const uint16_t* __restrict__ y,
                                                            const int32_t* __restrict__ slot, int32_t H,
                                                            int32_t Krt, float* __restrict__ grad_w) {
  __shared__ float wpart[kMaxWaves * kMaxK];
  const int K = KT > 0 ? KT : Krt;
  const uint32_t t = blockIdx.x;
  const uint32_t v = threadIdx.x;  // 8-channel vector
  const bool act = v < static_cast<uint32_t>(H) / 8;
  const int32_t* srow = slot + static_cast<size_t>(t) * K;

  // loaded by every lane (a lane past the last vector reads vector 0 and
  // zeroes it): a load under a per-lane condition is waited for before the
  // row gathers are issued, a memory latency of its own
  const u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(grad_out + static_cast<size_t>(t) * H) +
                                              (act ? v : 0u));
  float g[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g[2 * i] = act ? bf16_lo(gv[i]) : 0.0f;
    g[2 * i + 1] = act ? bf16_hi(gv[i]) : 0.0f;
  }
  if (KT > 0) {
    weights_chunk<(KT > 0 ? KT : 1)>(y, srow, 0, K, H, v, act, g, wpart);
  } else {
    for (int k0 = 0; k0 < K; k0 += 8) weights_chunk<8>(y, srow, k0, K, H, v, act, g, wpart);
  }
  __syncthreads();
  if (v < static_cast<uint32_t>(K)) {
    const int nw = blockDim.x / kWave;
    int len = 1;
    while (len < nw) len <<= 1;
    float a[kMaxWaves];
#pragma unroll
    for (int i = 0; i < kMaxWaves; ++i) a[i] = i < nw ? wpart[i * kMaxK + v] : -0.0f;
    for (; len > 1; len >>= 1)
#pragma unroll
      for (int i = 0; i < kMaxWaves / 2; ++i)
        if (i < len / 2) a[i] = __fadd_rn(a[2 * i], a[2 * i + 1]);
    grad_w[static_cast<size_t>(t) * K + v] = srow[v] >= 0 ? a[0] : 0.0f;
  }
}

}  // namespace

hipError_t launch_combine_backward(const uint16_t* grad_out, const uint16_t* y, const int32_t* slot,
                                   const float* w, int32_t T, int32_t H, int32_t K, uint16_t* grad_y,
                                   float* grad_w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const uint32_t vpt = static_cast<uint32_t>(H) / 8;
  const uint32_t n_items = static_cast<uint32_t>(T) * vpt;
  const dim3 rgrid((n_items + kRowThreads - 1) / kRowThreads), rblock(kRowThreads);
  const int lanes = (H / 8 + kWave - 1) / kWave * kWave;
  const dim3 wgrid(T), wblock(lanes);
  hipError_t e = hipSuccess;
  const bool burst = launch_fanout_burst_bf16(grad_out, slot, w, T, H, K, true, grad_y, nullptr, stream, &e);
  if (e != hipSuccess) return e;
#define EP_COMBINE_BWD(KV)                                                                                    \
  if (!burst)                                                                                                 \
    hipLaunchKernelGGL(grad_rows_kernel<KV>, rgrid, rblock, 0, stream, grad_out, slot, w, n_items, vpt, H, K, \
                       grad_y);                                                                               \
  if (grad_w != nullptr)                                                                                      \
    hipLaunchKernelGGL(grad_weights_kernel<KV>, wgrid, wblock, 0, stream, grad_out, y, slot, H, K, grad_w)
  switch (K) {
    case 1: { EP_COMBINE_BWD(1); } break;
    case 2: { EP_COMBINE_BWD(2); } break;
    case 4: { EP_COMBINE_BWD(4); } break;
    case 6: { EP_COMBINE_BWD(6); } break;
    case 8: { EP_COMBINE_BWD(8); } break;
    default: { EP_COMBINE_BWD(0); } break;
  }
#undef EP_COMBINE_BWD
  return hipGetLastError();
}

}  // namespace ep
