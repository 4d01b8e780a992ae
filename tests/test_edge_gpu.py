"""GPU edge cases against the oracle: empty, ragged and degenerate inputs,
runtime-K paths, layout path boundaries, and special values."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_U8, gpu_combine, gpu_dispatch, gpu_layout, host, to_dev
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def full_check(ep, idx, E, x_bits, y_bits=None, w=None, fp8=True):
    T, K = idx.shape
    print("case T=%d K=%d E=%d H=%d fp8=%s" % (T, K, E, x_bits.shape[1], fp8), flush=True)
    if w is None:
        w = np.random.default_rng(T * 31 + K).standard_normal((T, K)).astype(np.float32)
    counts, offsets, slot, src = gpu_layout(ep, idx, E)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_)
    assert np.array_equal(host(src), osrc)
    nv = int(oo[-1])
    if T == 0:
        return
    recv, scale, rw = gpu_dispatch(ep, x_bits, slot, w, fp8=fp8)
    if fp8:
        orecv, oscale, orw = oracle.dispatch_fp8(x_bits, os_, topk_weights=w)
        hr = host(recv)
        assert np.array_equal(hr[:nv], orecv[:nv])
        assert np.all(hr[nv:] == SENT_U8)
        assert np.array_equal(host(scale)[:nv].view(np.uint32), oscale[:nv].view(np.uint32))
    else:
        orecv = oracle.dispatch_bf16(x_bits, os_)
        orw = oracle.dispatch_fp8(x_bits, os_, topk_weights=w)[2] if x_bits.shape[1] % 128 == 0 else None
        assert np.array_equal(host(recv)[:nv], orecv[:nv])
    if orw is not None:
        assert np.array_equal(host(rw)[:nv], orw[:nv])
    if y_bits is None:
        y_bits = to_bf16_bits(np.random.default_rng(K).standard_normal((T * K, x_bits.shape[1]), dtype=np.float32))
    out = host(gpu_combine(ep, y_bits, slot, w))
    assert np.array_equal(out, oracle.combine(y_bits, os_, w))


def rand_x(T, H, seed=0):
    return to_bf16_bits(np.random.default_rng(seed).standard_normal((T, H), dtype=np.float32))


def test_empty_batch(gpu):
    idx = np.zeros((0, 8), np.int32)
    full_check(gpu, idx, 256, np.zeros((0, 7168), np.uint16))


@pytest.mark.parametrize("T", [1, 3, 37, 129])
def test_ragged_small(gpu, T):
    rng = np.random.default_rng(T)
    idx = np.argsort(rng.random((T, 256)), axis=1)[:, :8].astype(np.int32)
    full_check(gpu, idx, 256, rand_x(T, 7168, T))


@pytest.mark.parametrize("K", [1, 3, 5, 7, 12, 32])
def test_runtime_and_odd_topk(gpu, K):
    T, E = 203, 64
    rng = np.random.default_rng(K)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    full_check(gpu, idx, E, rand_x(T, 384, K))
    full_check(gpu, idx, E, rand_x(T, 72, K), fp8=False)


def test_duplicates_masks_and_out_of_range(gpu):
    rng = np.random.default_rng(5)
    T, K, E = 300, 6, 10
    idx = rng.integers(-3, E + 3, size=(T, K)).astype(np.int32)  # duplicates, -1..-3, >= E
    full_check(gpu, idx, E, rand_x(T, 256, 5))


def test_all_masked(gpu):
    idx = np.full((50, 4), -1, np.int32)
    full_check(gpu, idx, 8, rand_x(50, 128, 1))


def test_everything_to_one_expert_and_k_equals_e(gpu):
    T = 3000
    idx = np.full((T, 1), 17, np.int32)
    full_check(gpu, idx, 256, rand_x(T, 128, 2))
    idx = np.tile(np.arange(8, dtype=np.int32)[::-1], (T, 1))  # K == E, every expert every token
    full_check(gpu, idx, 8, rand_x(T, 128, 3))


@pytest.mark.parametrize("E", [1, 2, 255, 257, 1024])
def test_expert_counts(gpu, E):
    rng = np.random.default_rng(E)
    T, K = 700, min(E, 4)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32) if E > 1 else np.zeros((T, 1), np.int32)
    full_check(gpu, idx, E, rand_x(T, 256, E))


@pytest.mark.parametrize("rows,E", [(1024, 256), (1025, 256), (4095, 256), (32767, 256), (32768, 256),
                                    (65536, 256), (65537, 256), (131073, 256), (262144, 256),
                                    (1024, 512), (1025, 512), (32768, 512), (65536, 512),
                                    (1024, 1024), (1025, 1024), (32768, 1024), (65536, 1024), (65537, 1024), (700, 1),
                                    (5000, 1)])
def test_layout_path_boundaries(gpu, rows, E):
    """One workgroup up to 1024 entries, one fused launch up to 65536, then
    two launches over 4096-entry chunks; ragged last steps and chunks."""
    K = 8 if rows % 8 == 0 else 1
    T = rows // K
    rng = np.random.default_rng(rows)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    print("case layout rows", rows, E, flush=True)
    counts, offsets, slot, src = gpu_layout(gpu, idx, E)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, E)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_) and np.array_equal(host(src), osrc)


def special_groups(rng, n, first=0):
    """n groups of 128 channels (float32, exact in BF16 where it matters),
    group i of pattern (first + i) % 13: zeros; signed zeros; a wide
    dynamic range; BF16 subnormals; +-3e38; 448 with an E4M3 tie; 2^-140;
    1e-30 scale; amax exactly 2^-80 with channels down to the BF16
    subnormals (the quantiser's shared-reciprocal path); amax just below
    2^-80 (its plain-division path); E4M3 ties after division by s = 3;
    normals at 2^-79; plain normals."""
    out = np.empty((n, 128), np.float32)
    for i in range(n):
        g = rng.standard_normal(128).astype(np.float32)
        sign = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
        spread = (2.0 ** -rng.uniform(0.0, 53.0, 128)).astype(np.float32)
        p = (first + i) % 13
        if p == 0:
            g[:] = 0.0
        elif p == 1:
            g[:] = sign * np.float32(0.0)
        elif p == 2:
            g *= np.float32(1e-3)
            g[5] = 300.0
        elif p == 3:
            g *= np.float32(2.0 ** -130)
        elif p == 4:
            g = sign * np.float32(3.0e38)
        elif p == 5:
            g[:] = 448.0
            g[1::7] = 1.0625
        elif p == 6:
            g[:] = np.float32(2.0 ** -140)
        elif p == 7:
            g *= np.float32(1e-30)
        elif p == 8:
            g = sign * np.float32(2.0 ** -80) * spread
            g[3] = np.float32(2.0 ** -80)
        elif p == 9:
            g = sign * np.float32(float.fromhex("0x1.fep-81")) * spread
            g[3] = -np.float32(float.fromhex("0x1.fep-81"))
        elif p == 10:
            ties = np.array([1.0625, 1.1875, 1.3125, 1.5625, 1.9375, 4.5 / 512, 0.5625, 0.03125 * 1.0625], np.float32)
            g = sign * np.float32(3.0) * ties[np.arange(128) % ties.size]
            g[0] = 1344.0
        elif p == 11:
            g *= np.float32(2.0 ** -79)
        out[i] = g
    return out


def special_tokens(rng, T, H):
    return special_groups(rng, T * H // 128).reshape(T, H)


def test_special_values(gpu):
    """Zero groups, signed zeros, FP8-subnormal outputs, BF16 subnormal
    inputs, the 2^-126 scale floor, huge magnitudes, exact ties."""
    T, H = 16, 512
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = 0.0
    x[1, :128] = -0.0
    x[1, 128:256] = 0.0
    x[1, 200] = -0.0
    x[2, :128] *= np.float32(1e-3)   # wide dynamic range: many FP8 subnormals
    x[2, 0] = 300.0
    x[3, :] *= np.float32(2.0 ** -130)  # BF16 subnormals; s floored at 2^-126
    x[4, :] = np.float32(3.0e38) * np.sign(x[4, :])
    x[5, :128] = np.float32(448.0)
    x[5, 1] = np.float32(1.0625 * 448 / 448)  # E4M3 tie after division by s = 1
    x[6, :128] = np.float32(2.0 ** -140)
    x[7, :] = np.float32(1e-30) * x[7, :]
    x[8:12, :128] = special_groups(rng, 4, first=8)  # around amax = 2^-80, and E4M3 ties with s = 3
    xb = to_bf16_bits(x)
    idx = np.stack([np.arange(T) % 5, (np.arange(T) + 2) % 5], axis=1).astype(np.int32)
    w = rng.standard_normal((T, 2)).astype(np.float32)
    w[0] = [-0.0, 0.0]
    w[4] = [0.5, 0.25]  # keeps the huge row's weighted sum finite
    y = xb[np.repeat(np.arange(T), 2)]
    full_check(gpu, idx, 5, xb, y_bits=y, w=w)
    full_check(gpu, idx, 5, xb, y_bits=y, w=w, fp8=False)


@pytest.mark.parametrize("rows", [900, 1800, 70000])
def test_masked_ids_of_every_value(gpu, rows):
    """Masked ids take many values (-1, -2, INT_MIN, E, INT_MAX): each must
    land in the masked bucket on every layout path (regression: a skip
    sentinel equal to a legal masked id once dropped entries from the count
    of masked rows)."""
    E = 16
    rng = np.random.default_rng(rows)
    idx = rng.integers(0, E, size=rows).astype(np.int64)
    bad = rng.random(rows) < 0.3
    idx[bad] = rng.choice([-1, -2, -3, E, E + 5, -(2 ** 31), 2 ** 31 - 1], size=int(bad.sum()))
    idx = idx.astype(np.int32).reshape(-1, 1)
    print("case masked ids rows", rows, flush=True)
    counts, offsets, slot, src = gpu_layout(gpu, idx, E)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, E)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_) and np.array_equal(host(src), osrc)


@pytest.mark.parametrize("rows", [1030, 9999, 40000])
def test_layout_unaligned_ids(gpu, rows):
    """topk_idx only 4-byte aligned: the fused path falls back from 16-byte
    to 4-byte id loads; same results."""
    rng = np.random.default_rng(rows + 1)
    idx = rng.integers(-1, 256, size=(rows, 1)).astype(np.int32)
    print("case unaligned ids rows", rows, flush=True)
    counts, offsets, slot, src = gpu_layout(gpu, idx, 256, misalign=True)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, 256)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_) and np.array_equal(host(src), osrc)


def test_debug_check_rejects_ids_outside_minus_one_to_e(gpu, monkeypatch):
    """With EP_DEBUG_CHECK on, the binding refuses ids outside [-1, E)
    before any launch; -1 (masked) passes, and with the check off the same
    ids are masked by the kernels."""
    import combine_ep_dispatch_amd.api as api
    ep = gpu
    E = 16
    idx = np.array([[0, 5], [-1, 15], [3, 16]], dtype=np.int32)
    print("case debug check", flush=True)
    monkeypatch.setattr(api, "DEBUG_CHECK", True)
    with pytest.raises(ValueError, match="EP_DEBUG_CHECK"):
        gpu_layout(ep, idx, E)
    counts, offsets, slot, src = gpu_layout(ep, idx[:2], E)  # only -1 out of range: accepted
    assert np.array_equal(host(slot), oracle.dispatch_layout(idx[:2], E)[2])
    monkeypatch.setattr(api, "DEBUG_CHECK", False)
    counts, offsets, slot, src = gpu_layout(ep, idx, E)  # 16 is masked
    assert np.array_equal(host(slot), oracle.dispatch_layout(idx, E)[2])


@pytest.mark.parametrize("T,H,scale_offset,K", [(300, 7168, 0, 8), (300, 7168, 1, 8), (300, 2048, 3, 8),
                                                 (300, 1536, 0, 8), (300, 512, 0, 8), (300, 2048, 0, 10),
                                                 (300, 1024, 1, 10), (1200, 7168, 0, 8), (1200, 7168, 1, 8),
                                                 (1200, 7168, 0, 10), (6000, 1536, 0, 8)])
def test_scale_store_paths(gpu, T, H, scale_offset, K):
    """FP8 scales are written 32 bytes per row by each wavefront when H is a
    multiple of 1024 and recv_scale is 16-byte aligned, else one lane per
    group: both against the oracle, the second forced by a recv_scale that
    starts scale_offset floats past an aligned address.  From 16 MB of tokens
    (T=1200 at 7168, T=6000 at 1536) the stores are non-temporal.  K=10 takes
    the kernel that walks a token's entries 8 at a time; the received
    weights ride along in every case."""
    ep = gpu
    rng = np.random.default_rng(T + H + scale_offset + K)
    E = 64
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    w = rng.random((T, K), dtype=np.float32)
    x = rand_x(T, H, seed=H)
    print("case scale stores T=%d H=%d offset=%d K=%d" % (T, H, scale_offset, K), flush=True)
    counts, offsets, slot, src = gpu_layout(ep, idx, E)
    R, G = T * K, H // 128
    recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
    store = torch.full((R * G + 4,), -3.0, dtype=torch.float32, device="cuda")
    scale = store[scale_offset:scale_offset + R * G].view(R, G)
    assert (scale.data_ptr() % 16 == 0) == (scale_offset == 0)
    rw = torch.full((R,), -5.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(to_dev(x.view(np.int16)), slot, to_dev(w), ep.EP_RECV_FP8_E4M3_G128, recv, scale, rw)
    oc, oo, oslot, osrc = oracle.dispatch_layout(idx, E)
    orecv, oscale, orw = oracle.dispatch_fp8(x, oslot, topk_weights=w)
    nv = int(oo[-1])
    assert np.array_equal(host(recv)[:nv], orecv[:nv])
    assert np.array_equal(host(scale)[:nv].view(np.uint32), oscale[:nv].view(np.uint32))
    assert np.array_equal(host(rw)[:nv].view(np.uint32), orw[:nv].view(np.uint32))
    assert np.all(host(rw)[nv:] == -5.0)
    # nothing written outside the scale rows of valid entries
    rest = host(store)
    assert np.all(rest[:scale_offset] == -3.0) and np.all(rest[scale_offset + nv * G:] == -3.0)


@pytest.mark.parametrize("T,H", [(16, 512), (128, 7168), (1000, 7168), (4096, 7168)])
def test_special_values_one_call(gpu, T, H):
    """The special-value groups through ep_layout_dispatch on each of its
    kernels: the decode kernel (16 and 128 tokens), the chunked kernel
    (1000 tokens) and the split kernel (4096 tokens of hidden 7168)."""
    from tests.test_chunked_gpu import routing, run_and_check
    rng = np.random.default_rng(T + H)
    idx = routing(rng, T, 8, 256, mask_frac=0.02)
    xb = to_bf16_bits(special_tokens(rng, T, H))
    w = rng.standard_normal((T, 8)).astype(np.float32)
    print("case special values one call T=%d H=%d" % (T, H), flush=True)
    run_and_check(gpu, idx, xb, w, 256, 0, True)
    run_and_check(gpu, idx, xb, w, 256, 40 if T >= 1000 else 4, True)
