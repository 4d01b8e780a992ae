"""Hardware-operation parity on gfx950: the binary32 -> E4M3FN conversion
and the binary32 division the FP8 dispatch relies on."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import gpu_dispatch, gpu_layout, host
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def test_cast_sweep_rounding_band(gpu):
    """Every binary32 with |v| in [2^-12, 2^10) (both signs) through the
    kernel's conversion vs the oracle's encoder; tails sampled."""
    ep = gpu
    for be in range(127 - 12, 127 + 10):
        bits = (np.uint32(be) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)
        v = bits.view(np.float32)
        want = oracle.f32_to_e4m3_rne_sat(v)
        for sign in (1, -1):
            vin = torch.from_numpy(v * np.float32(sign)).cuda()
            out = torch.empty(vin.shape, dtype=torch.uint8, device="cuda")
            ep.ep_cast_fp8_e4m3(vin, out)
            got = host(out)
            exp = want if sign == 1 else want | np.uint8(0x80)
            bad = np.flatnonzero(got != exp)
            assert bad.size == 0, (be, sign, v[bad[:4]], got[bad[:4]], exp[bad[:4]])
    rng = np.random.default_rng(1)
    tails = np.concatenate([
        rng.integers(0, (127 - 12) << 23, 1 << 20, dtype=np.uint64),
        rng.integers((127 + 10) << 23, 0x7F800000, 1 << 20, dtype=np.uint64),
        np.array([0, 1, 0x7F7FFFFF, 0x43E00000, 0x43E00001, 0x43E80000], dtype=np.uint64),
    ]).astype(np.uint32)
    v = np.concatenate([tails, tails | np.uint32(0x80000000)]).view(np.float32)
    # odd length exercises the tail path of the cast kernel
    v = v[:-1]
    vin = torch.from_numpy(v).cuda()
    out = torch.empty(vin.shape, dtype=torch.uint8, device="cuda")
    ep.ep_cast_fp8_e4m3(vin, out)
    assert np.array_equal(host(out), oracle.f32_to_e4m3_rne_sat(v))


def test_cast_tails_exhaustive(gpu):
    """Every finite binary32 outside the band above, both signs: below 2^-12
    the code is a signed zero, from 2^10 up it saturates to +-448 (0x7E).
    The oracle's encoder gives exactly these codes on the sampled tails of
    the previous test; here all ~3.9e9 inputs are generated and compared on
    the device, in chunks.  With the band above this covers every finite
    binary32 (NaN and infinity are outside the contract)."""
    ep = gpu
    band_lo, band_hi, inf_bits = (127 - 12) << 23, (127 + 10) << 23, 0x7F800000
    chunk = 1 << 28
    for start, stop, code in ((0, band_lo, 0x00), (band_hi, inf_bits, 0x7E)):
        for a in range(start, stop, chunk):
            b = min(stop, a + chunk)
            bits = torch.arange(a, b, dtype=torch.int64, device="cuda").to(torch.int32)
            for sign in (0, 1):
                v = (bits | torch.tensor(-(2 ** 31), dtype=torch.int32, device="cuda")) if sign else bits
                out = torch.empty(b - a, dtype=torch.uint8, device="cuda")
                ep.ep_cast_fp8_e4m3(v.view(torch.float32), out)
                want = code | (sign << 7)
                bad = torch.nonzero(out != want)
                assert bad.numel() == 0, (hex(a), sign, hex(int(bits[bad[0, 0]])), int(out[bad[0, 0]]), hex(want))
            del bits, v, out
    torch.cuda.synchronize()


def division_sensitive_groups(n_groups=512, seed=4):
    """Groups whose quotients x/s sit on or next to E4M3 midpoints, where a
    reciprocal-multiply or a wrongly rounded division flips the code."""
    rng = np.random.default_rng(seed)
    groups = []
    while len(groups) < n_groups:
        amax = to_bf16_bits(np.array([rng.uniform(1.0, 400.0)], np.float32))
        amax_f = oracle.bf16_bits_to_f32(amax)[0]
        s = np.float32(amax_f / np.float32(448.0))
        cand = np.arange(0x3C00, int(amax[0]), dtype=np.uint16)
        xf = oracle.bf16_bits_to_f32(cand)
        qd = (xf / s).astype(np.float32)
        qm = (xf * np.float32(np.float32(1.0) / s)).astype(np.float32)
        diff = np.flatnonzero(oracle.f32_to_e4m3_rne_sat(qd) != oracle.f32_to_e4m3_rne_sat(qm))
        if diff.size == 0:
            continue
        g = np.empty(128, np.uint16)
        g[0] = amax[0]
        g[1:] = cand[rng.choice(diff, size=127)]
        g[1:] ^= rng.integers(0, 2, 127).astype(np.uint16) << 15  # random signs
        groups.append(g)
    return np.stack(groups)


def test_division_sensitive_dispatch(gpu):
    ep = gpu
    g = division_sensitive_groups()
    x = g.reshape(-1, 1024)  # 8 groups per token
    T = x.shape[0]
    idx = np.zeros((T, 1), np.int32)
    print("case division-sensitive T=%d" % T, flush=True)
    _, _, slot, _ = gpu_layout(ep, idx, 1)
    recv, scale, _ = gpu_dispatch(ep, x, slot, None)
    _, _, oslot, _ = oracle.dispatch_layout(idx, 1)
    orecv, oscale, _ = oracle.dispatch_fp8(x, oslot)
    assert np.array_equal(host(scale).view(np.uint32), oscale.view(np.uint32))
    assert np.array_equal(host(recv), orecv)
