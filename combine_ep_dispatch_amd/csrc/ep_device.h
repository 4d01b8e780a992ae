// Device-side helpers shared by the dispatch-layout, dispatch and combine
// kernels (gfx950, wave64).  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ep {

constexpr int kWave = 64;
constexpr int kGroup = 128;  // channels per FP8 scale group

// LDS one workgroup may allocate on gfx950: the CU's whole 160 KB.
constexpr size_t kLdsLimit = 160 * 1024;

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

// Inclusive prefix sum over the 64 lanes of a wavefront, with DPP: shifts
// by 1, 2, 4 and 8 inside each 16-lane row (lanes without a source add 0),
// then row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds the total of rows 0-1 to rows 2 and 3.  Integer
// addition, so the order of the partial sums does not matter.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive prefix sum of data[0..n) in LDS, in place, by wave 0 alone:
// each lane sums ceil(n/64) consecutive values, the lanes' sums are scanned
// across the wave, and each lane rewrites its run.  Every thread of the
// block must call it (it ends with the barrier that publishes the result).
// MAXPER bounds ceil(n/64): the lane's values stay in registers.
template <int MAXPER>
__device__ inline void block_exclusive_scan_upto(int* data, int n) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (n + kWave - 1) / kWave;
    const int beg = lane * per;
    int v[MAXPER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      v[i] = (i < per && beg + i < n) ? data[beg + i] : 0;
      local += v[i];
    }
    int run = wave_inclusive_scan(local) - local;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (i < per && beg + i < n) data[beg + i] = run;
      run += v[i];
    }
  }
  __syncthreads();
}

// n <= 17 * 64 (up to 1024 experts and the masked key)
__device__ inline void block_exclusive_scan(int* data, int n) {
  if (n <= 5 * kWave) block_exclusive_scan_upto<5>(data, n);
  else if (n <= 9 * kWave) block_exclusive_scan_upto<9>(data, n);
  else block_exclusive_scan_upto<17>(data, n);
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

// RN32(a / b) for a BF16 value a, given y = RN32(1 / b): q0 = RN32(|a| y),
// then one FMA correction with the residual |a| - q0 b, and a's sign put
// back (so -0 stays -0).  Checked exhaustively on the CPU against IEEE
// division: every BF16 significand over two binades against every binary32
// significand of b, 2^31 pairs, all correctly rounded.  The check carries
// over to other exponents while |a| >= 2^-102 and 2^-126 <= b < 2^126:
// the residual is then either exact or of magnitude >= 2^-125, so it rounds
// as it does in the checked binades.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
  const float x = __builtin_fabsf(a);
  const float q0 = x * y;
  const float r0 = __builtin_fmaf(-q0, b, x);
  return __builtin_copysignf(__builtin_fmaf(r0, y, q0), a);
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

  // The quotients by the shared s: one correctly rounded reciprocal, then a
  // multiply and an FMA correction per channel (div_by_recip).  Channels
  // below 2^-102 fall outside its check; with amax >= 2^-80 their quotient
  // is below 448 * 2^-22 < 2^-10, which is E4M3 +-0 however it rounds.
  // A group with 0 < amax < 2^-80 takes the plain division.
  u32x4 q;
  if (m != 0 && m < 0x17800000u) {  // 2^-80
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = f32x4_to_e4m3(f[4 * j] / s, f[4 * j + 1] / s, f[4 * j + 2] / s, f[4 * j + 3] / s);
  } else {
    const float y = 1.0f / s;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = f32x4_to_e4m3(div_by_recip(f[4 * j], s, y), div_by_recip(f[4 * j + 1], s, y),
                           div_by_recip(f[4 * j + 2], s, y), div_by_recip(f[4 * j + 3], s, y));
  }
  scale = s;
  return q;
}

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled by construction:
// registers held in arrays (a lane's token vectors) must be indexed by
// constants, and an index the compiler does not resolve puts the array in
// scratch memory (`#pragma unroll` is only a request).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---- dispatch stores ------------------------------------------------------

// One 16-byte token load; NT: non-temporal (a token read once).
template <bool NT>
__device__ __forceinline__ u32x4 load_token(const u32x4* p) {
  return NT ? __builtin_nontemporal_load(p) : *p;
}

// The 8 group scales one wavefront of FP8 work items covers (64 lanes of 16
// channels: 8 whole 128-channel groups of one token, lanes 0, 8, .., 56
// holding them after quantize16_e4m3), written 32 bytes per receive row:
// each lane with a row (rj >= 0, one lane per row of the token, loaded by
// that lane itself: a select among the lanes' copies would be turned into
// an indexed array in LDS) stores all 8 to row rj.  v is this lane's work
// item in the token, G = H/128; the 32-byte pieces must be 16-byte aligned
// (G a multiple of 4, recv_scale 16-byte aligned).  Every lane of the
// wavefront must call it.
template <bool NT>
__device__ __forceinline__ void store_wave_scales(int32_t rj, float s, uint32_t v, uint32_t G,
                                                  float* __restrict__ recv_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  u32x4 lo, hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = __builtin_amdgcn_readlane(__float_as_uint(s), 8 * i);
    hi[i] = __builtin_amdgcn_readlane(__float_as_uint(s), 8 * (i + 4));
  }
  if (rj >= 0) {
    u32x4* dst = reinterpret_cast<u32x4*>(recv_scale + static_cast<size_t>(rj) * G + ((v - lane) >> 3));
    if (NT) {
      __builtin_nontemporal_store(lo, dst);
      __builtin_nontemporal_store(hi, dst + 1);
    } else {
      dst[0] = lo;
      dst[1] = hi;
    }
  }
}

}  // namespace ep
