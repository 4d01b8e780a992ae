"""Tolerances of the parity tests that are not bit-exact (CPU helpers, no
torch, no oracle import).

grad_w, the weight gradient of combine, is a dot product over H channels.
The oracle gives the exact dot product rounded once to binary32; the GPU
sums its binary32 products in an order of its own choosing.  The library
states how deep that order is: every product is exact (a BF16 x BF16
product has a 16-bit significand), and each product then passes through at
most 7 + ceil(log2(H/8)) binary32 additions (8-channel partial sums, then
a tree over the H/8 partial sums).  Recursive summation with at most n
rounded additions on any term's path is within gamma_n * sum|p_i| of the
exact sum (gamma_n = n*u / (1 - n*u), u = 2^-24; Higham, "Accuracy and
Stability of Numerical Algorithms", section 4.2), and the oracle's one
rounding adds at most u * |sum| <= u * sum|p_i|.  So

    |grad_w_gpu - grad_w_oracle| <= (8 + ceil(log2(H/8))) * u * (1 + 2^-16) * sum_c |g_c * y_c|
                                    + H * 2^-150

where the last term covers products that fall below the normal binary32
range (each then rounded by at most half the smallest subnormal).
"""

import math

import numpy as np

U32 = 2.0 ** -24


def _widen(bits):
    """BF16 bits -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def grad_w_depth(H):
    """Rounded additions on any product's path, plus the oracle's rounding."""
    return 8 + int(math.ceil(math.log2(max(1, H // 8))))


def grad_w_bound(g_bits, y_bits, slot, chunk=1024):
    """Per-(t, k) bound on |GPU grad_w - oracle grad_w| (0 for masked
    entries, which must be +0.0 exactly).  g_bits uint16[T, H], y_bits
    uint16[rows, H], slot int32[T, K]."""
    g = np.asarray(g_bits, dtype=np.uint16)
    yb = np.asarray(y_bits, dtype=np.uint16)
    slot = np.asarray(slot)
    T, K = slot.shape
    H = g.shape[1]
    scale = grad_w_depth(H) * U32 * (1.0 + 2.0 ** -16)
    out = np.zeros((T, K), dtype=np.float64)
    for t0 in range(0, T, chunk):
        gt = np.abs(_widen(g[t0:t0 + chunk]))
        for k in range(K):
            r = slot[t0:t0 + chunk, k].astype(np.int64)
            m = r >= 0
            mag = (gt[m] * np.abs(_widen(yb[r[m]]))).sum(axis=1)
            col = np.zeros(r.shape[0])
            col[m] = scale * mag + H * 2.0 ** -150
            out[t0:t0 + chunk, k] = col
    return out


def assert_grad_w_close(got, want, bound, slot):
    """GPU grad_w against the oracle's: within the bound, masked entries
    +0.0 bit for bit."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    masked = np.asarray(slot) < 0
    assert np.all(got[masked].view(np.uint32) == 0), "masked entries must be +0.0"
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = np.argwhere(~(diff <= bound))
    assert bad.size == 0, "grad_w outside the bound at %s: got %r want %r bound %r" % (
        bad[:4].tolist(), got[tuple(bad[0])], want[tuple(bad[0])], bound[tuple(bad[0])])
