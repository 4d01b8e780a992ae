"""GPU parity: the HIP path against the oracle on every workload.

Bar: layout, indices, FP8 bytes, scales and routing weights bit-exact; the
combine output bit-exact as well (the arithmetic is fixed, so any
difference is a defect; the contract's 1-BF16-ulp tolerance is asserted
separately as the documented bound).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import (SENT_BF16, SENT_F32, SENT_U8, gpu_combine, gpu_dispatch, gpu_layout, host,
                           to_dev)
from workloads import make_workload

pytestmark = pytest.mark.gpu


def check_layout(ep, wl):
    counts, offsets, slot, src = gpu_layout(ep, wl.topk_idx, wl.E)
    oc, oo, os_, osrc = oracle.dispatch_layout(wl.topk_idx, wl.E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_)
    assert np.array_equal(host(src), osrc)
    return slot, oo, os_


def assert_bf16_within_one_ulp(got, want):
    g = oracle.bf16_bits_to_f32(got).astype(np.float64)
    w = oracle.bf16_bits_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - w) <= np.abs(w) * 2.0 ** -7 + 1e-38)


@pytest.mark.parametrize("name,seed,over", [("tiny", 0, {}), ("tiny", 1, {}), ("tiny", 2, {}), ("decode", 0, {}),
                                            ("decode", 1, {}), ("decode", 2, {}), ("prefill", 0, {}),
                                            ("prefill", 1, {}), ("skew", 0, {}), ("skew", 1, {}),
                                            ("skew", 2, {"holes_frac": 0.25})])
def test_fp8_workload_parity(gpu, name, seed, over):
    """over: config overrides; holes_frac=0.25 gives a quarter of the
    experts zero popularity (empty experts under skew)."""
    ep = gpu
    wl = make_workload(name, seed=seed, **over)
    print("case", name, seed, flush=True)
    slot, off, oslot = check_layout(ep, wl)
    nv = int(off[-1])
    recv, scale, rw = gpu_dispatch(ep, wl.x_bits, slot, wl.topk_weights)
    orecv, oscale, orw = oracle.dispatch_fp8(wl.x_bits, oslot, topk_weights=wl.topk_weights)
    assert np.array_equal(host(recv)[:nv], orecv[:nv])
    assert np.array_equal(host(scale)[:nv].view(np.uint32), oscale[:nv].view(np.uint32))
    assert np.array_equal(host(rw)[:nv], orw[:nv])
    out = host(gpu_combine(ep, wl.y_bits, slot, wl.topk_weights))
    oout = oracle.combine(wl.y_bits, oslot, wl.topk_weights)
    assert_bf16_within_one_ulp(out, oout)
    assert np.array_equal(out, oout)


def test_hbm_bf16_full_size(gpu):
    """T=32768, H=7168, BF16 dispatch (3.76 GB receive buffer) + combine on
    the receive buffer itself (identity expert), every output compared:
    the receive rows against the oracle's BF16 dispatch, and all 32768 x
    7168 combine outputs against the oracle's combine of the oracle's
    receive rows, 1024 tokens at a time."""
    ep = gpu
    wl = make_workload("hbm", seed=0)
    print("case hbm 0", flush=True)
    slot, off, oslot = check_layout(ep, wl)
    nv = int(off[-1])
    d_x = to_dev(wl.x_bits.view(np.int16))
    recv, _, _ = gpu_dispatch(ep, d_x, slot, None, fp8=False)
    oy = oracle.dispatch_bf16(wl.x_bits, oslot)
    assert np.array_equal(host(recv)[:nv], oy[:nv])
    w = to_dev(wl.topk_weights)
    out = host(gpu_combine(ep, recv, slot, w))
    del recv
    print("case hbm 0: combine outputs", flush=True)
    for t0 in range(0, wl.T, 1024):
        t1 = min(wl.T, t0 + 1024)
        want = oracle.combine(oy, oslot[t0:t1], wl.topk_weights[t0:t1])
        assert np.array_equal(out[t0:t1], want), "tokens %d..%d" % (t0, t1)


def test_prefill_fp8_then_bf16_combine_of_dequantised_rows(gpu):
    """Round trip at the prefill size: FP8 dispatch, dequantise (oracle),
    combine on the GPU == oracle combine, and within the FP8 bound of x."""
    ep = gpu
    wl = make_workload("prefill", seed=2)
    print("case prefill roundtrip", flush=True)
    slot, off, oslot = check_layout(ep, wl)
    recv, scale, _ = gpu_dispatch(ep, wl.x_bits, slot)
    y = oracle.dequantize_rows(host(recv), host(scale))
    out = host(gpu_combine(ep, y, slot, wl.topk_weights))
    assert np.array_equal(out, oracle.combine(y, oslot, wl.topk_weights))
    x = oracle.bf16_bits_to_f32(wl.x_bits).astype(np.float64)
    s_el = np.repeat(oracle.quantize_tokens_fp8(wl.x_bits)[1], 128, axis=1).astype(np.float64)
    o = oracle.bf16_bits_to_f32(out).astype(np.float64)
    assert np.all(np.abs(o - x) <= 0.071 * np.abs(x) + 2.0 ** -9 * s_el)


def test_untouched_rows_and_determinism(gpu):
    """Masked entries leave rows past expert_offset[E] untouched; repeated
    runs are bit-identical (skew routing, multi-block layout)."""
    ep = gpu
    wl = make_workload("skew", seed=2, T=2048)
    idx = wl.topk_idx.copy()
    idx[::7, 3] = -1
    idx[::11, 5] = 999
    print("case masked skew", flush=True)
    c1, o1, s1, r1 = gpu_layout(ep, idx, wl.E)
    c2, o2, s2, r2 = gpu_layout(ep, idx, wl.E)
    for a, b in ((c1, c2), (o1, o2), (s1, s2), (r1, r2)):
        assert torch.equal(a, b)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, wl.E)
    assert np.array_equal(host(s1), os_) and np.array_equal(host(r1), osrc)
    nv = int(oo[-1])
    recv, scale, rw = gpu_dispatch(ep, wl.x_bits, s1, wl.topk_weights)
    recv2, scale2, rw2 = gpu_dispatch(ep, wl.x_bits, s1, wl.topk_weights)
    assert torch.equal(recv, recv2) and torch.equal(scale, scale2) and torch.equal(rw, rw2)
    hr, hs, hw = host(recv), host(scale), host(rw)
    assert np.all(hr[nv:] == SENT_U8) and np.all(hs[nv:] == SENT_F32) and np.all(hw[nv:] == SENT_F32)
    orecv, oscale, orw = oracle.dispatch_fp8(wl.x_bits, os_, topk_weights=wl.topk_weights)
    assert np.array_equal(hr[:nv], orecv[:nv]) and np.array_equal(hs[:nv], oscale[:nv])
    y = wl.y_bits
    out1 = gpu_combine(ep, y, s1, wl.topk_weights)
    out2 = gpu_combine(ep, y, s1, wl.topk_weights)
    assert torch.equal(out1, out2)
    assert np.array_equal(host(out1), oracle.combine(y, os_, wl.topk_weights))
    assert not np.any(host(out1) == SENT_BF16)
