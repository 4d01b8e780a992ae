"""Pins for the oracle's BF16 and FP8 E4M3FN codecs (CPU only)."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f32, e4m3_to_f32, f32_to_bf16_rne, f32_to_e4m3_rne_sat
from tests.pins import E4M3_POS, e4m3_encode_exact, e4m3_table_encoder, e4m3_value


def enc1(v):
    return int(f32_to_e4m3_rne_sat(np.array([v], dtype=np.float32))[0])


# Closed-form values from the OCP 8-bit floating point specification v1.0,
# E4M3 table: bias 7, max normal S.1111.110 = 448, min normal S.0001.000 =
# 2**-6, min subnormal S.0000.001 = 2**-9, NaN S.1111.111, no infinities.
@pytest.mark.parametrize("value,code", [
    (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E),
    (-448.0, 0xFE), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (-(2.0 ** -9), 0x81),
    (7 * 2.0 ** -9, 0x07), (1.875 * 2.0 ** 7, 0x77), (1.125, 0x39), (0.5, 0x30),
])
def test_e4m3_spec_points(value, code):
    assert enc1(value) == code
    assert float(e4m3_to_f32(np.array([code], dtype=np.uint8))[0]) == value or (value == 0 and code in (0, 0x80))


def test_e4m3_saturation_and_ties():
    # beyond the largest finite value everything saturates (satfinite)
    for v in (448.0001, 464.0, 480.0, 1e6, 3.0e38):
        assert enc1(v) == 0x7E and enc1(-v) == 0xFE
    # ties between neighbouring codes go to the even code
    assert enc1(1.0 + 1 / 16) == 0x38      # between 0x38 (1.0) and 0x39 (1.125): even is 0x38
    assert enc1(1.125 + 1 / 16) == 0x3A    # between 0x39 and 0x3A: even is 0x3A
    assert enc1(2.0 ** -10) == 0x00        # half of the smallest subnormal: tie to 0
    assert enc1(3 * 2.0 ** -10) == 0x02    # between 0x01 and 0x02
    assert enc1(416.0) == 0x7D             # 1.625 * 2**8 is a code of its own
    assert enc1(432.0) == 0x7E             # between 416 (0x7D) and 448 (0x7E): even is 0x7E
    assert enc1(400.0) == 0x7C             # between 384 (0x7C) and 416 (0x7D): even is 0x7C
    assert enc1(15 * 2.0 ** -10) == 0x08   # between 7*2**-9 (0x07) and 2**-6 (0x08)
    # just off a tie rounds to the nearer code
    assert enc1(np.nextafter(np.float32(1.0 + 1 / 16), np.float32(2))) == 0x39
    assert enc1(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01


def test_e4m3_bytes_read_as_torch_float8():
    """The receive bytes are OCP E4M3FN, the encoding of torch's
    float8_e4m3fn: all 256 codes, viewed as that dtype, decode to the
    oracle's values (the two NaN codes to NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    via_torch = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = e4m3_to_f32(codes)
    nan = np.isnan(ours)
    assert np.array_equal(np.isnan(via_torch), nan) and nan.sum() == 2
    assert np.array_equal(via_torch[~nan].view(np.uint32), ours[~nan].view(np.uint32))


def test_e4m3_tails_are_constant():
    """Outside [2**-12, 2**10) the code depends only on the sign: below 2**-12
    a value is under half the smallest subnormal (2**-10), so it rounds to
    a signed zero; from 2**10 up it is beyond 448, so it saturates.  Random
    bit patterns from both tails (the GPU test sweeps them all on the
    device against exactly these constants)."""
    rng = np.random.default_rng(3)
    lo = rng.integers(0, (127 - 12) << 23, 200_000, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers((127 + 10) << 23, 0x7F800000, 200_000, dtype=np.uint64).astype(np.uint32)
    sign = np.uint32(0x80000000)
    assert np.all(f32_to_e4m3_rne_sat(lo.view(np.float32)) == 0x00)
    assert np.all(f32_to_e4m3_rne_sat((lo | sign).view(np.float32)) == 0x80)
    assert np.all(f32_to_e4m3_rne_sat(hi.view(np.float32)) == 0x7E)
    assert np.all(f32_to_e4m3_rne_sat((hi | sign).view(np.float32)) == 0xFE)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    dec = e4m3_to_f32(codes)
    for c in range(256):
        ref = e4m3_value(c)
        if ref is None:
            assert math.isnan(dec[c])
        else:
            assert Fraction(float(dec[c])) == ref


def test_e4m3_exact_rational_random():
    """Random binary32 values across the whole code range vs exact rounding."""
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-14, 10, size=4000)).astype(np.float32)
    signs = rng.choice([-1.0, 1.0], size=mags.size).astype(np.float32)
    vals = mags * signs
    got = f32_to_e4m3_rne_sat(vals)
    for v, g in zip(vals, got):
        assert int(g) == e4m3_encode_exact(Fraction(float(v))), float(v)


def test_e4m3_exact_rational_ties_and_neighbours():
    """Every midpoint between adjacent codes, and its two float32 neighbours."""
    pts = []
    for i in range(len(E4M3_POS) - 1):
        mid = np.float32(float((E4M3_POS[i] + E4M3_POS[i + 1]) / 2))
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    vals = np.array(pts, dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    got = f32_to_e4m3_rne_sat(vals)
    for v, g in zip(vals, got):
        assert int(g) == e4m3_encode_exact(Fraction(float(v))), float(v)


def test_e4m3_sweep_vs_table_encoder():
    """Every binary32 pattern with |v| in [2**-12, 2**10) vs the table encoder.

    Below 2**-12 everything rounds to a signed zero and above 448 everything
    saturates; both tails are sampled.  Sign symmetry is checked on a stride.
    """
    table = e4m3_table_encoder()
    lo_exp, hi_exp = 127 - 12, 127 + 10
    for be in range(lo_exp, hi_exp):
        bits = (np.uint32(be) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)
        v = bits.view(np.float32)
        got = f32_to_e4m3_rne_sat(v)
        want = table(v)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (be, v[bad[:5]], got[bad[:5]], want[bad[:5]])
        neg = f32_to_e4m3_rne_sat(-v[::97])
        assert np.array_equal(neg, want[::97] | np.uint8(0x80))
    rng = np.random.default_rng(3)
    tiny = (rng.integers(0, lo_exp << 23, size=200000, dtype=np.uint64)).astype(np.uint32).view(np.float32)
    assert np.array_equal(f32_to_e4m3_rne_sat(tiny), np.zeros(tiny.size, np.uint8))
    assert np.all(f32_to_e4m3_rne_sat(-tiny - np.float32(0)) == 0x80)
    huge = (rng.integers(hi_exp << 23, 0x7F800000, size=200000, dtype=np.uint64)).astype(np.uint32).view(np.float32)
    assert np.all(f32_to_e4m3_rne_sat(huge) == 0x7E)


def test_e4m3_vs_torch_cast():
    """Black-box cross-check: torch's CPU float8_e4m3fn cast (RNE) in range."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(500000) * np.exp2(rng.uniform(-12, 8, 500000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3_rne_sat(v), ref)


def test_bf16_vs_torch_cast():
    """Random finite binary32 patterns and exact ties vs torch's CPU bf16 cast."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    ties = ((rng.integers(0, 0x7F7F, 100000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.array([0.0, -0.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(v), ref)


def test_bf16_widen_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (f.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(f) & np.isnan(ref))
    assert same.all()


def test_bf16_rne_hand_ties():
    # 1 + 2**-8 is halfway between bf16 1.0 and 1 + 2**-7: even is 1.0
    assert int(f32_to_bf16_rne(np.array([1 + 2 ** -8], np.float32))[0]) == 0x3F80
    # 1 + 3*2**-8 is halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    assert int(f32_to_bf16_rne(np.array([1 + 3 * 2 ** -8], np.float32))[0]) == 0x3F82
    assert int(f32_to_bf16_rne(np.array([-0.0], np.float32))[0]) == 0x8000
