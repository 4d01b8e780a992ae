// Device-side helpers shared by the dispatch-layout, dispatch and combine
// kernels (gfx950, wave64).  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;
constexpr int kGroup = 128;  // channels per FP8 scale group

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- wavefront primitives -------------------------------------------------

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// Number of set bits of `mask` in lanes strictly below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Max over the 8 aligned lanes 8j..8j+7 of non-negative binary32 values held
// as their bit patterns (for non-negative IEEE values integer order equals
// numeric order, so the max is exact).  Three DPP steps inside a row:
// swap neighbours, swap pairs, then mirror the half-row.
__device__ __forceinline__ uint32_t max8_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// The key of an expert id (int32 or int64): the id itself inside [0, E),
// otherwise E (a masked entry).  Every kernel turns ids into keys as it
// loads them, so wide ids never meet 32-bit arithmetic.
template <typename Idx>
__device__ __forceinline__ int expert_key(Idx e, int E) {
  return (e >= 0 && e < static_cast<Idx>(E)) ? static_cast<int>(e) : E;
}

// Keys of the 16 / sizeof(Idx) consecutive ids held in one 16-byte load
// (little-endian: an int64 id is the dword pair lo, hi).
template <typename Idx>
__device__ __forceinline__ void expert_keys16(const int4 v, int E, int* key) {
  if constexpr (sizeof(Idx) == 4) {
    key[0] = expert_key(v.x, E);
    key[1] = expert_key(v.y, E);
    key[2] = expert_key(v.z, E);
    key[3] = expert_key(v.w, E);
  } else {
    static_assert(sizeof(Idx) == 8, "ids are int32 or int64");
    const auto join = [](int lo, int hi) {
      return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                  static_cast<uint32_t>(lo));
    };
    key[0] = expert_key(join(v.x, v.y), E);
    key[1] = expert_key(join(v.z, v.w), E);
  }
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive prefix sum of data[0..n) in LDS, in place.  Every thread of the
// block must call it.  wave_tot needs blockDim.x / 64 ints of LDS.
__device__ inline void block_exclusive_scan(int* data, int n, int* wave_tot) {
  const int tid = threadIdx.x, bs = blockDim.x;
  const int lane = tid & (kWave - 1), w = tid / kWave, nw = bs / kWave;
  const int per = (n + bs - 1) / bs;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  int local = 0;
  for (int i = beg; i < end; ++i) local += data[i];
  const int incl = wave_inclusive_scan(local);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int v = lane < nw ? wave_tot[lane] : 0;
    const int s = wave_inclusive_scan(v);
    if (lane < nw) wave_tot[lane] = s - v;
  }
  __syncthreads();
  int run = wave_tot[w] + incl - local;
  for (int i = beg; i < end; ++i) {
    const int c = data[i];
    data[i] = run;
    run += c;
  }
  __syncthreads();
}

// ---- number formats -------------------------------------------------------

// BF16 bits in the low / high half of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> BF16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four binary32 values -> four OCP E4M3FN bytes (little-endian in a word),
// round to nearest even.  gfx950's v_cvt_pk_fp8_f32 converts to the OCP
// encoding; inputs are clamped to +-448 first so the result saturates at the
// largest finite code instead of producing NaN (v_med3 keeps -0.0 and every
// in-range value unchanged).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// One lane's 16 consecutive channels (two 16-byte vectors of BF16 bits) ->
// 16 E4M3 codes, and the binary32 scale of their 128-channel group, which
// the 8 aligned lanes 8j..8j+7 hold together (all 8 must call this).
// Scale rule: s = RN32(amax / 448) with a correctly rounded division, 1 for
// an all-zero group, floored at 2^-126; code = E4M3_RNE(RN32(x / s)).
__device__ __forceinline__ u32x4 quantize16_e4m3(u32x4 a, u32x4 b, float& scale) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(a[i]);
    f[2 * i + 1] = bf16_hi(a[i]);
    f[8 + 2 * i] = bf16_lo(b[i]);
    f[8 + 2 * i + 1] = bf16_hi(b[i]);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  m = max8_u32(m);  // all 8 lanes of the group now hold its |max| bits

  float s = __uint_as_float(m) / 448.0f;
  s = s < 0x1p-126f ? 0x1p-126f : s;
  s = m == 0 ? 1.0f : s;

  u32x4 q;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    q[j] = f32x4_to_e4m3(f[4 * j] / s, f[4 * j + 1] / s, f[4 * j + 2] / s, f[4 * j + 3] / s);
  scale = s;
  return q;
}

}  // namespace ep
