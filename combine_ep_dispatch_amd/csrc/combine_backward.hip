// Backward of combine: gradients w.r.t. the expert outputs and the routing
// weights ([P5 "典型工作流程"] lists backward helpers beside combine; the
// pages give no arithmetic for them).
//
// combine computes out[t] = sum_k w[t,k] * y[slot[t,k]], so
//   grad_y[slot[t,k], c] = BF16_RNE(RN32(w[t,k] * grad_out[t,c]))
//   grad_w[t,k]          = sum_c grad_out[t,c] * y[slot[t,k], c]
// The dot product has a fixed order, so results are reproducible and
// bit-identical to the definition: the 8 products of each 8-channel vector
// are added in channel order into +0.0, then the H/8 vector sums are added
// as a complete binary tree of adjacent pairs, padded with -0.0 (an exact
// identity for addition).
//
// gfx950 design: one workgroup per token, one lane per 8 channels (H <=
// 8192).  Each lane loads its grad_out vector once and the K expert-row
// vectors (non-temporal, read once), writes K grad_y vectors (plain stores:
// scattered rows, as in dispatch) and forms K vector sums.  A wave reduces
// them with a butterfly over lanes (xor 1, 2, ..., 32: step d adds the
// blocks of d adjacent leaves, i.e. the adjacent-pair tree), and lane 0 of
// each wave parks its sums in LDS; K lanes then finish the tree over the
// waves.  HBM-bound: per token 2H + 2KH bytes in, 2KH + 4K out.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMaxWaves = 16;  // workgroups of up to 1024 lanes
constexpr int kMaxK = 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_tree_sum(float x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x = __fadd_rn(x, __shfl_xor(x, d, kWave));
  return x;
}

template <int KC>
__device__ __forceinline__ void backward_chunk(const uint16_t* __restrict__ y, const int32_t* __restrict__ srow,
                                               const float* __restrict__ wrow, int k0, int K, int32_t H, uint32_t v,
                                               bool act, bool want_w, const float (&g)[8],
                                               uint16_t* __restrict__ grad_y, float* wpart) {
  int32_t r[KC];
  float wk[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const bool in = k0 + j < K;
    r[j] = in ? srow[k0 + j] : -1;
    wk[j] = in ? wrow[k0 + j] : 0.0f;
  }
  u32x4 d[KC];
  if (want_w) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      d[j] = u32x4{0, 0, 0, 0};
      if (act && r[j] >= 0)
        d[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + static_cast<size_t>(r[j]) * H) + v);
    }
  }
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (act && r[j] >= 0) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_rne(__fmul_rn(wk[j], g[2 * i])) | (f32_to_bf16_rne(__fmul_rn(wk[j], g[2 * i + 1])) << 16);
      reinterpret_cast<u32x4*>(grad_y + static_cast<size_t>(r[j]) * H)[v] = o;
    }
    if (want_w && k0 + j < K) {
      float part = -0.0f;  // lanes past the last vector are tree padding
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
}

template <int KT>
__global__ __launch_bounds__(1024) void combine_backward_kernel(const uint16_t* __restrict__ grad_out,
                                                                const uint16_t* __restrict__ y,
                                                                const int32_t* __restrict__ slot,
                                                                const float* __restrict__ w, int32_t H, int32_t Krt,
                                                                uint16_t* __restrict__ grad_y,
                                                                float* __restrict__ grad_w) {
  __shared__ float wpart[kMaxWaves * kMaxK];
  const int K = KT > 0 ? KT : Krt;
  const uint32_t t = blockIdx.x;
  const uint32_t v = threadIdx.x;  // 8-channel vector
  const bool act = v < static_cast<uint32_t>(H) / 8;
  const bool want_w = grad_w != nullptr;
  const int32_t* srow = slot + static_cast<size_t>(t) * K;
  const float* wrow = w + static_cast<size_t>(t) * K;

  float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (act) {
    const u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(grad_out + static_cast<size_t>(t) * H) + v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[2 * i] = bf16_lo(gv[i]);
      g[2 * i + 1] = bf16_hi(gv[i]);
    }
  }
  if (KT > 0) {
    backward_chunk<(KT > 0 ? KT : 1)>(y, srow, wrow, 0, K, H, v, act, want_w, g, grad_y, wpart);
  } else {
    for (int k0 = 0; k0 < K; k0 += 8) backward_chunk<8>(y, srow, wrow, k0, K, H, v, act, want_w, g, grad_y, wpart);
  }
  if (!want_w) return;
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
  const int lanes = (H / 8 + kWave - 1) / kWave * kWave;
  const dim3 grid(T), block(lanes);
#define EP_COMBINE_BWD(KV)                                                                                  \
  hipLaunchKernelGGL(combine_backward_kernel<KV>, grid, block, 0, stream, grad_out, y, slot, w, H, K, grad_y, \
                     grad_w)
  switch (K) {
    case 1: EP_COMBINE_BWD(1); break;
    case 2: EP_COMBINE_BWD(2); break;
    case 4: EP_COMBINE_BWD(4); break;
    case 6: EP_COMBINE_BWD(6); break;
    case 8: EP_COMBINE_BWD(8); break;
    default: EP_COMBINE_BWD(0); break;
  }
#undef EP_COMBINE_BWD
  return hipGetLastError();
}

}  // namespace ep
