// Device-side helpers shared by the dispatch-layout, dispatch and combine
// kernels (gfx950, wave64).  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;
constexpr int kGroup = 128;  // channels per FP8 scale group

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

}  // namespace ep
