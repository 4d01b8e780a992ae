"""Independent reference formulations used to pin the oracle.

Nothing here imports ``oracle``; each function restates a definition in a
different form (exact rationals, brute-force counting, a lookup table) so
that a slip in the oracle's vectorised code shows up as a disagreement.
"""

import math
from fractions import Fraction

import numpy as np

F32_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)


def f32_frac(v):
    """Exact rational value of a float (binary32 or binary64)."""
    return Fraction(float(v))


def rn32(fr):
    """Round an exact rational to the nearest binary32, ties to even.

    Returns a Python float holding the binary32 value (inf on overflow).
    Zero results are returned as +0.0; callers handle the sign of zero.
    """
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)  # below 2**-126 the spacing stays 2**-149
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r > F32_MAX:
        # round-to-nearest overflows to infinity beyond max + half ulp
        return -math.inf if neg else math.inf
    return -float(r) if neg else float(r)


def f32_mul(a, b):
    """IEEE binary32 multiply (RNE) with the IEEE sign-of-zero rule."""
    r = rn32(f32_frac(a) * f32_frac(b))
    if r == 0.0:
        neg = (math.copysign(1.0, a) < 0) != (math.copysign(1.0, b) < 0)
        return -0.0 if neg else 0.0
    return r


def f32_add(a, b):
    """IEEE binary32 add (RNE): an exact zero sum is +0 unless both are -0."""
    r = rn32(f32_frac(a) + f32_frac(b))
    if r == 0.0:
        both_neg = math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0
        return -0.0 if both_neg else 0.0
    return r


def f32_div(a, b):
    """IEEE binary32 divide (RNE) for finite a and nonzero finite b."""
    r = rn32(f32_frac(a) / f32_frac(b))
    if r == 0.0:
        neg = (math.copysign(1.0, a) < 0) != (math.copysign(1.0, b) < 0)
        return -0.0 if neg else 0.0
    return r


# ---- OCP E4M3FN, from the specification's value formula -------------------

def e4m3_value(code):
    """Exact value of an E4M3FN code as a Fraction (None for NaN)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 2 ** 9)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_POS = [e4m3_value(c) for c in range(0x7F)]  # codes 0x00..0x7E, ascending


def e4m3_encode_exact(fr, negative_zero=False):
    """Nearest E4M3FN code to an exact rational, ties to the even code,
    magnitudes beyond 448 saturate to 0x7E."""
    neg = fr < 0 or (fr == 0 and negative_zero)
    a = -fr if fr < 0 else fr
    if a >= E4M3_POS[-1]:
        code = 0x7E
    else:
        # first code whose value is >= a
        hi = next(c for c in range(0x7F) if E4M3_POS[c] >= a)
        if E4M3_POS[hi] == a or hi == 0:
            code = hi
        else:
            lo = hi - 1
            dlo, dhi = a - E4M3_POS[lo], E4M3_POS[hi] - a
            if dlo < dhi:
                code = lo
            elif dhi < dlo:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi
    return code | (0x80 if neg else 0)


def e4m3_table_encoder():
    """Vectorised table encoder: returns f(x_nonneg float32 array) -> codes.

    Builds the sorted table of the 127 finite non-negative code values and
    their midpoints (exact in float64) and rounds by binary search; a value
    exactly on a midpoint takes the even code.
    """
    vals = np.array([float(v) for v in E4M3_POS], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0

    def enc(x):
        x = np.asarray(x, dtype=np.float64)
        lo = np.searchsorted(mids, x, side="left")
        hi = np.searchsorted(mids, x, side="right")
        tie = lo != hi
        code = np.where(tie, np.where(lo % 2 == 0, lo, hi), lo)
        return code.astype(np.uint8)

    return enc


# ---- layout by brute-force counting ----------------------------------------

def brute_layout(topk_idx, E):
    """Direct counting definition of the stable expert-major layout.

    slot[t][k] = (number of valid entries whose expert is smaller)
               + (number of entries of the same expert that come earlier in
                  (t, k) order).  Masked entries (expert outside [0, E))
    get -1; src lists tokens row by row with -1 past the valid rows.
    """
    T = len(topk_idx)
    K = len(topk_idx[0]) if T else 0
    entries = [(t, k, int(topk_idx[t][k])) for t in range(T) for k in range(K)]
    valid = [(t, k, e) for (t, k, e) in entries if 0 <= e < E]
    counts = [sum(1 for (_, _, e) in valid if e == x) for x in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    slot = [[-1] * K for _ in range(T)]
    for (t, k, e) in valid:
        below = sum(1 for (_, _, e2) in valid if e2 < e)
        earlier = sum(1 for (t2, k2, e2) in valid if e2 == e and (t2, k2) < (t, k))
        slot[t][k] = below + earlier
    src = [-1] * (T * K)
    for (t, k, e) in valid:
        src[slot[t][k]] = t
    return counts, offsets, slot, src


def brute_layout_padded(topk_idx, E, cap):
    """Padded layout by counting: rank = earlier (t, k) entries with the
    same expert; kept when rank < cap, at row e*cap + rank."""
    T = len(topk_idx)
    K = len(topk_idx[0]) if T else 0
    slot = [[-1] * K for _ in range(T)]
    seen = [0] * E
    src = [-1] * (E * cap)
    for t in range(T):
        for k in range(K):
            e = int(topk_idx[t][k])
            if not 0 <= e < E:
                continue
            r = seen[e]
            seen[e] += 1
            if r < cap:
                slot[t][k] = e * cap + r
                src[e * cap + r] = t
    return [min(c, cap) for c in seen], slot, src
