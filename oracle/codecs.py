"""Number-format codecs used by the oracle (test infrastructure only).

The pages name the formats but not their encodings: dispatch travels in FP8
and combine returns BF16 ([P1] "DeepEP 的常规内核和低延迟内核"; FP8 support
is listed under "DeepEP 的核心功能").  The encodings below are the public
definitions:

* BF16: the upper 16 bits of an IEEE-754 binary32; rounding from binary32
  is round-to-nearest, ties-to-even (RNE).
* FP8 E4M3FN (OCP 8-bit floating point specification v1.0): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 encodes
  subnormals M * 2**-9.  There is no infinity; S.1111.111 is NaN, so the
  largest finite magnitude is 0x7E = 1.75 * 2**8 = 448.  Conversion from
  binary32 rounds to nearest, ties to even, and saturates finite values
  beyond 448 to +-448 ("satfinite").

Everything is integer bit manipulation on numpy arrays so that no host
library rounding is involved.  Non-finite inputs are outside the method's
domain and are rejected.
"""

import numpy as np

E4M3_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits):
    """Widen BF16 bit patterns (uint16) to float32.  Exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(v):
    """Round float32 values to BF16 (RNE); returns uint16 bit patterns.

    Adding 0x7FFF plus the lowest kept bit and truncating implements
    round-half-to-even on the 16 discarded bits; a carry out of the
    mantissa correctly bumps the exponent (and reaches the infinity
    pattern for values beyond the BF16 range, as IEEE RNE prescribes).
    """
    f = np.ascontiguousarray(v, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("non-finite value outside the oracle's domain")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_e4m3_rne_sat(v):
    """Encode float32 values as OCP E4M3FN bytes, RNE with saturation.

    Returns uint8 codes.  Signed zero keeps its sign (-0.0 -> 0x80).
    """
    f = np.ascontiguousarray(v, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("non-finite value outside the oracle's domain")
    u = f.view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1) << 7
    a = u & 0x7FFFFFFF  # magnitude bits
    biased_exp = a >> 23  # binary32 exponent field
    out = np.zeros(a.shape, dtype=np.int64)

    # |v| >= 448: saturate.  448 = 0x43E00000.
    sat = a >= 0x43E00000

    # 2**-6 <= |v| < 448: the FP8 value is normal.  Keep 3 of the 23
    # mantissa bits with round-half-even on the 20 dropped ones, then move
    # the exponent bias from 127 to 7 (subtract 120 << 3 from the shifted
    # pattern).  A carry into the exponent is handled by the addition.
    normal = (~sat) & (biased_exp >= 127 - 6)
    keep = (a >> 20) & 1
    rn = (a + 0x7FFFF + keep) >> 20
    code_n = rn - (120 << 3)
    out = np.where(normal, np.minimum(code_n, 0x7E), out)

    # |v| < 2**-6: the FP8 value is subnormal, M * 2**-9 with M in 0..8
    # (M == 8 is the smallest normal, code 0x08, which the same integer
    # happens to encode).  M = RNE(|v| * 2**9) computed on the integer
    # significand: |v| = sig * 2**(e - 150) for a normal binary32 with
    # biased exponent e, so |v| * 2**9 = sig >> (141 - e).
    small = (~sat) & (~normal)
    sig = np.where(biased_exp > 0, (a & 0x7FFFFF) | 0x800000, a & 0x7FFFFF)
    e_eff = np.where(biased_exp > 0, biased_exp, 1)
    shift = 141 - e_eff  # >= 21 here because e <= 120
    big_shift = shift > 40  # result certainly 0 (sig < 2**24)
    sh = np.where(big_shift, 40, shift)
    q = sig >> sh
    rem = sig & ((np.int64(1) << sh) - 1)
    half = np.int64(1) << (sh - 1)
    up = (rem > half) | ((rem == half) & ((q & 1) == 1))
    m = np.where(big_shift, 0, q + up.astype(np.int64))
    out = np.where(small, m, out)

    out = np.where(sat, 0x7E, out)
    return (out | sign).astype(np.uint8)


def e4m3_to_f32(codes):
    """Decode OCP E4M3FN bytes to float32 (exact).  NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (s * mag).astype(np.float32)
