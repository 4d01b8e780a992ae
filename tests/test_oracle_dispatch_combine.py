"""Pins for the oracle's FP8/BF16 dispatch and its combine (CPU only)."""

import math

import numpy as np
import pytest

from oracle import (bf16_bits_to_f32, combine, dequantize_rows, dispatch_bf16, dispatch_fp8,
                    dispatch_layout, e4m3_to_f32, quantize_tokens_fp8)
from tests.pins import (e4m3_encode_exact, f32_add, f32_div, f32_frac, f32_mul, rn32)
from workloads import make_workload, to_bf16_bits


def exact_quantize_group(xs):
    """Quantise one 128-channel group with exact rationals + explicit RN32."""
    a = max(abs(float(v)) for v in xs)
    if a == 0:
        s = 1.0
    else:
        s = rn32(f32_frac(a) / 448)
        s = max(s, 2.0 ** -126)
    codes = []
    for v in xs:
        q = f32_div(float(v), s)
        codes.append(e4m3_encode_exact(f32_frac(q), negative_zero=math.copysign(1.0, q) < 0))
    return codes, s


def test_quantiser_exact_rational_small():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal((3, 256)) * np.exp2(rng.uniform(-20, 6, (3, 1)))).astype(np.float32)
    x32[1, :128] = 0.0
    x32[1, 5] = -0.0
    x32[2, 128:] *= np.float32(2.0 ** -120)  # a group needing the 2**-126 scale floor
    xb = to_bf16_bits(x32)
    q, s = quantize_tokens_fp8(xb)
    xf = bf16_bits_to_f32(xb)
    for t in range(3):
        for g in range(2):
            codes, sg = exact_quantize_group(xf[t, 128 * g:128 * (g + 1)])
            assert float(s[t, g]) == sg, (t, g)
            assert q[t, 128 * g:128 * (g + 1)].tolist() == codes, (t, g)


def test_quantiser_invariants_decode():
    wl = make_workload("decode", seed=1)
    q, s = quantize_tokens_fp8(wl.x_bits)
    xf = bf16_bits_to_f32(wl.x_bits).reshape(wl.T, -1, 128)
    a = np.abs(xf).max(axis=2)
    qg = q.reshape(wl.T, -1, 128)
    # the group maximum lands on the top code (448) in every nonzero group
    assert np.all(((qg & 0x7F) == 0x7E).any(axis=2)[a > 0])
    # s*448 is within one ulp of amax
    ulp = np.spacing(a.astype(np.float32))
    assert np.all(np.abs(s.astype(np.float64) * 448 - a) <= ulp)
    # dequantised error: E4M3 half-spacing is 2**-4 relative for normal codes,
    # 2**-10 * s absolute in the subnormal band
    deq = e4m3_to_f32(q).reshape(wl.T, -1, 128).astype(np.float64) * s[:, :, None]
    err = np.abs(deq - xf)
    assert np.all(err <= np.abs(xf) * 2.0 ** -4 * (1 + 2.0 ** -20) + s[:, :, None] * 2.0 ** -10)


def test_dispatch_fans_out_identical_copies():
    wl = make_workload("tiny", seed=3)
    _, offsets, slot, src = dispatch_layout(wl.topk_idx, wl.E)
    recv, scale, rw = dispatch_fp8(wl.x_bits, slot, topk_weights=wl.topk_weights)
    q, s = quantize_tokens_fp8(wl.x_bits)
    for r in range(offsets[-1]):
        t = src[r]
        assert np.array_equal(recv[r], q[t]) and np.array_equal(scale[r], s[t])
    for t in range(wl.T):
        for k in range(wl.K):
            assert rw[slot[t, k]] == wl.topk_weights[t, k]
    rb = dispatch_bf16(wl.x_bits, slot)
    assert np.array_equal(rb[: offsets[-1]], wl.x_bits[src[: offsets[-1]]])


def emulated_combine(yb, slot, w):
    """The ordered binary32 weighted sum, one element at a time, with exact
    rationals and explicit IEEE rounding (tests/pins.py)."""
    T, K = slot.shape
    H = yb.shape[1]
    yf = bf16_bits_to_f32(yb)
    out = np.empty((T, H), np.float32)
    for t in range(T):
        for c in range(H):
            acc = 0.0
            for k in range(K):
                r = slot[t, k]
                if r < 0:
                    continue
                acc = f32_add(acc, f32_mul(float(w[t, k]), float(yf[r, c])))
            out[t, c] = acc
    return out


def test_combine_exact_emulation_tiny():
    wl = make_workload("tiny", seed=0)
    _, _, slot, _ = dispatch_layout(wl.topk_idx, wl.E)
    yb = wl.y_bits
    # add cancellation, signed zeros and a masked pick
    w = wl.topk_weights.copy()
    w[0, :] = [0.5, -0.5]
    yb = yb.copy()
    yb[slot[0, 1]] = yb[slot[0, 0]]
    w[1, 0] = -0.0
    slot = slot.copy()
    slot[2, 1] = -1
    T = 12
    got = combine(yb, slot[:T], w[:T])
    acc = emulated_combine(yb, slot[:T], w[:T])
    import torch
    want = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert np.all(got[0] == 0)  # exact cancellation gives +0.0


def test_combine_k1_identity():
    rng = np.random.default_rng(4)
    T, H = 50, 64
    yb = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    slot = rng.permutation(T).astype(np.int32)[:, None]
    out = combine(yb, slot, np.ones((T, 1), np.float32))
    assert np.array_equal(out, yb[slot[:, 0]])


def test_combine_vs_float64_bound_decode():
    wl = make_workload("decode", seed=0)
    _, _, slot, _ = dispatch_layout(wl.topk_idx, wl.E)
    got = bf16_bits_to_f32(combine(wl.y_bits, slot, wl.topk_weights)).astype(np.float64)
    yf = bf16_bits_to_f32(wl.y_bits).astype(np.float64)
    w = wl.topk_weights.astype(np.float64)
    terms = w[:, :, None] * yf[slot]
    exact = terms.sum(axis=1)
    mag = np.abs(terms).sum(axis=1)
    # K roundings of binary32 (2**-24 each, relative to the running magnitude)
    # plus one BF16 rounding of the result (2**-8 relative, half an ulp)
    bound = wl.K * 2.0 ** -24 * mag + np.abs(exact) * 2.0 ** -8 + 2.0 ** -133
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9))


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("skew", 256)])
def test_round_trip_identity_expert(name, T):
    """dispatch -> identity expert -> combine with weights summing to 1
    reproduces x within the FP8 quantisation bound."""
    wl = make_workload(name, seed=0, T=T)
    _, offsets, slot, _ = dispatch_layout(wl.topk_idx, wl.E)
    recv, scale, _ = dispatch_fp8(wl.x_bits, slot)
    y = dequantize_rows(recv, scale)
    out = bf16_bits_to_f32(combine(y, slot, wl.topk_weights)).astype(np.float64)
    x = bf16_bits_to_f32(wl.x_bits).astype(np.float64)
    s_el = np.repeat(quantize_tokens_fp8(wl.x_bits)[1], 128, axis=1).astype(np.float64)
    assert np.all(np.abs(out - x) <= 0.071 * np.abs(x) + 2.0 ** -9 * s_el)


def test_round_trip_bf16_dispatch():
    wl = make_workload("tiny", seed=1)
    _, _, slot, _ = dispatch_layout(wl.topk_idx, wl.E)
    y = dispatch_bf16(wl.x_bits, slot)
    out = bf16_bits_to_f32(combine(y, slot, wl.topk_weights)).astype(np.float64)
    x = bf16_bits_to_f32(wl.x_bits).astype(np.float64)
    # sum of w is 1 within float32 rounding: at most one BF16 ulp away
    assert np.all(np.abs(out - x) <= np.abs(x) * 2.0 ** -7 + 1e-38)


def test_quantiser_uses_true_division():
    """Inputs where x * RN(1/s) and RN(x / s) fall on different E4M3 codes.

    A seeded search over BF16 group maxima and BF16 channel values finds
    quotients that sit on (or one binary32 ulp from) an E4M3 midpoint; on
    those a reciprocal-multiply quantiser picks the other code.  The oracle
    must agree with the exact-rational division on every one.
    """
    rng = np.random.default_rng(9)
    found = 0
    for _ in range(200):
        amax_bits = int(to_bf16_bits(np.array([rng.uniform(1.0, 400.0)], np.float32))[0])
        amax = float(bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
        s = rn32(f32_frac(amax) / 448)
        recip = rn32(1 / f32_frac(s))
        # every positive BF16 value below amax in a few binades
        cand = np.arange(0x3C00, amax_bits, dtype=np.uint16)
        xf = bf16_bits_to_f32(cand).astype(np.float64)
        q_div = (xf.astype(np.float32) / np.float32(s)).astype(np.float32)
        q_mul = (xf.astype(np.float32) * np.float32(recip)).astype(np.float32)
        from oracle import f32_to_e4m3_rne_sat as enc
        diff = np.flatnonzero(enc(q_div) != enc(q_mul))
        for i in diff[:3]:
            group = np.zeros(128, np.uint16)
            group[0] = amax_bits
            group[1] = cand[i]
            q, sg = quantize_tokens_fp8(group[None, :])
            codes, s_exact = exact_quantize_group(bf16_bits_to_f32(group))
            assert float(sg[0, 0]) == s_exact
            assert q[0].tolist() == codes
            assert int(q[0, 1]) == int(enc(q_div[i:i + 1])[0]) != int(enc(q_mul[i:i + 1])[0])
            found += 1
    assert found >= 5


def test_combine_order_sensitive_cases():
    """Sums built so that ascending-k binary32 accumulation, any other order,
    and exact accumulation give three different BF16 results' worth of
    disagreement: [b, half a BF16 ulp of b, 0.4 binary32 ulp, 0.4 binary32
    ulp].  Ascending keeps the exact tie (rounds to even); descending or
    exact summation leaves the tie and rounds away."""
    rng = np.random.default_rng(12)
    cases = []
    for _ in range(64):
        e = int(rng.integers(-20, 20))
        mant = int(rng.integers(0, 64)) * 2  # even 7-bit BF16 mantissa
        b = (1 + mant / 128) * 2.0 ** e
        half_bf16 = 2.0 ** (e - 8)
        small = 0.4 * 2.0 ** (e - 23)
        cases.append([b, half_bf16, small, small])
    vals = np.array(cases, np.float32)  # exact: every term is a binary32
    T, K = vals.shape
    # y = 1.0 everywhere; the terms ride in the weights (products exact)
    w = vals.copy()
    yb = to_bf16_bits(np.ones((T * K, 1), np.float32))
    slot = np.arange(T * K, dtype=np.int32).reshape(T, K)
    got = combine(yb, slot, w)
    emu = emulated_combine(yb, slot, w)
    import torch
    want = torch.from_numpy(emu).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # discriminating: exact real summation rounds differently on every case
    exact = vals.astype(np.float64).sum(axis=1).astype(np.float32)
    exact_b = torch.from_numpy(exact[:, None]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.all(exact_b != got)
    rev = combine(yb, slot[:, ::-1].copy(), w[:, ::-1].copy())
    assert np.all(rev != got)
