/* The FP8 quantiser's division by a shared scale (div_by_recip in
 * csrc/ep_device.h), checked on the CPU against IEEE binary32 division:
 *
 *   y = RN(1/b);  q0 = RN(|a| y);  r0 = RN(|a| - q0 b) (fma);
 *   q1 = RN(q0 + r0 y) (fma);  result = copysign(q1, a)
 *
 * 1. Exhaustive over significands: a every BF16 value in [1, 4) (two
 *    binades, so the quotient crosses 1 both ways), b every binary32 value
 *    in [1, 2): q1 must equal a / b in every pair.  The uncorrected q0 is
 *    counted too, so that a check which could not fail shows up.
 * 2. Sampled over exponents: |a| >= 2^-102 with a binary32 quotient in the
 *    normal range, b in [2^-126, 2^126): q1 == |a| / b.
 * 3. Channels below 2^-102 in a group with amax >= 2^-80 (b = RN(amax /
 *    448)): the quotient stays below 2^-10, where E4M3 rounds to zero.
 * 4. Signed zeros: -0 / b gives -0.
 *
 * Prints "pairs P q0_wrong W0 q1_wrong W1 sampled S sample_wrong W2 tiny T
 * tiny_wrong W3 zero_wrong W4"; exit status 0 when W1 = W2 = W3 = W4 = 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t f2u(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float div_by_recip(float a, float b, float y) {
  const float x = fabsf(a);
  const float q0 = x * y;
  const float r0 = fmaf(-q0, b, x);
  return copysignf(fmaf(r0, y, q0), a);
}

/* splitmix64 */
static uint64_t sm_state = 0x243F6A8885A308D3ull;
static uint64_t next64(void) {
  uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main(void) {
  long pairs = 0, q0_wrong = 0, q1_wrong = 0;
  for (uint32_t ab = 0; ab < 256; ++ab) {
    const float a = u2f((0x3F80u + ab) << 16);
    for (uint32_t bm = 0; bm < (1u << 23); ++bm) {
      const float b = u2f(0x3F800000u | bm);
      volatile float vy = 1.0f / b;
      const float y = vy;
      const float want = a / b;
      const float q0 = a * y;
      ++pairs;
      q0_wrong += f2u(q0) != f2u(want);
      q1_wrong += f2u(div_by_recip(a, b, y)) != f2u(want);
    }
  }

  long sampled = 0, sample_wrong = 0;
  while (sampled < 20000000) {
    const uint64_t r = next64();
    const int ea = -102 + (int)(r % 230);               /* 2^-102 .. 2^127 */
    const int eb = -126 + (int)((r >> 8) % 252);        /* 2^-126 .. 2^125 */
    const uint32_t am = (uint32_t)(r >> 16) & 0x7Fu;     /* BF16 fraction */
    const uint32_t bm = (uint32_t)(r >> 24) & 0x7FFFFFu;
    if (ea > 127) continue;
    const float a = u2f(((uint32_t)(ea + 127) << 23) | (am << 16));
    const float b = u2f(((uint32_t)(eb + 127) << 23) | bm);
    const float want = a / b;
    if (!(fabsf(want) >= 0x1p-126f) || isinf(want)) continue;
    volatile float vy = 1.0f / b;
    ++sampled;
    sample_wrong += f2u(div_by_recip(a, b, vy)) != f2u(want);
  }

  long tiny = 0, tiny_wrong = 0;
  for (int i = 0; i < 2000000; ++i) {
    const uint64_t r = next64();
    /* amax: a BF16 value in [2^-80, 2^127]; a: a BF16 value below 2^-102 */
    const int em = -80 + (int)(r % 208);
    const float amax = u2f(((uint32_t)(em + 127) << 23) | ((uint32_t)(r >> 8) & 0x7Fu) << 16);
    const uint32_t abits = (uint32_t)(r >> 20) & 0xFFFFu;
    const float a = u2f(abits << 16);
    if (!(fabsf(a) < 0x1p-102f)) continue;
    float s = amax / 448.0f;
    if (s < 0x1p-126f) s = 0x1p-126f;
    volatile float vy = 1.0f / s;
    ++tiny;
    const float q = div_by_recip(a, s, vy);
    tiny_wrong += !(fabsf(q) < 0x1p-10f) || (signbit(q) != signbit(a));
  }

  long zero_wrong = 0;
  {
    const float bs[3] = {0x1p-126f, 1.0f, 0x1.fffffep125f};
    for (int i = 0; i < 3; ++i) {
      volatile float vy = 1.0f / bs[i];
      zero_wrong += f2u(div_by_recip(-0.0f, bs[i], vy)) != 0x80000000u;
      zero_wrong += f2u(div_by_recip(0.0f, bs[i], vy)) != 0u;
    }
  }

  printf("pairs %ld q0_wrong %ld q1_wrong %ld sampled %ld sample_wrong %ld tiny %ld tiny_wrong %ld zero_wrong %ld\n",
         pairs, q0_wrong, q1_wrong, sampled, sample_wrong, tiny, tiny_wrong, zero_wrong);
  return (q1_wrong || sample_wrong || tiny_wrong || zero_wrong) ? 1 : 0;
}
