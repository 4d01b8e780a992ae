"""ep_layout_dispatch (layout and dispatch in one call) against the oracle.

Bar: every output bit-exact, rows and entries the contract leaves alone
still hold their sentinels.  Cases span the decode kernel (up to 3072
entries) and the paths beyond it (the chunked kernel has its own file),
packed and padded layouts, FP8 and BF16, masked ids of every kind, generic
top-k, ragged hidden sizes and the empty batch.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, SENT_F32, SENT_I32, SENT_U8, host, to_dev
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


def run_fused(ep, idx, x_bits, w, E, cap, fp8, with_weight=True):
    T, K = idx.shape
    H = x_bits.shape[1]
    R = E * cap if cap else T * K
    d_idx = to_dev(idx.astype(np.int32))
    d_x = to_dev(x_bits.view(np.int16))
    d_w = to_dev(w.astype(np.float32)) if w is not None else None
    counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    offsets = None if cap else torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((R,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda") if nb else None
    if fp8:
        recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
        scale = torch.full((R, H // 128), SENT_F32, dtype=torch.float32, device="cuda")
        fmt = ep.EP_RECV_FP8_E4M3_G128
    else:
        recv = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
        scale = None
        fmt = ep.EP_RECV_BF16
    rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda") if (with_weight and w is not None) else None
    ep.ep_layout_dispatch(d_idx, d_x, d_w if rw is not None else None, E, cap, fmt, counts, offsets, slot, src,
                          recv, scale, rw, ws)
    return counts, offsets, slot, src, recv, scale, rw


def check_fused(ep, idx, x_bits, w, E, cap=0, fp8=True, with_weight=True):
    T, K = idx.shape
    H = x_bits.shape[1]
    counts, offsets, slot, src, recv, scale, rw = run_fused(ep, idx, x_bits, w, E, cap, fp8, with_weight)
    if cap:
        oc, oslot, osrc = oracle.dispatch_layout_padded(idx, E, cap)
        used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
        R = E * cap
        assert np.array_equal(host(counts), oc)
        assert np.array_equal(host(slot), oslot)
        hs = host(src)
        assert np.array_equal(hs[used], osrc[used]) and np.all(hs[~used] == SENT_I32)
    else:
        oc, oo, oslot, osrc = oracle.dispatch_layout(idx, E)
        R = T * K
        used = np.arange(R) < oo[-1]
        assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
        assert np.array_equal(host(slot), oslot)
        assert np.array_equal(host(src), osrc)
    if T == 0:
        return
    if fp8:
        orecv, oscale, orw = oracle.dispatch_fp8(x_bits, oslot, num_rows=R, topk_weights=w)
        hr, hs = host(recv), host(scale)
        assert np.array_equal(hr[used], orecv[used]) and np.all(hr[~used] == SENT_U8)
        assert np.array_equal(hs[used].view(np.uint32), oscale[used].view(np.uint32))
        assert np.all(hs[~used] == SENT_F32)
    else:
        orecv = oracle.dispatch_bf16(x_bits, oslot, num_rows=R)
        hr = host(recv)
        assert np.array_equal(hr[used], orecv[used]) and np.all(hr[~used] == SENT_BF16)
        # the routing weights ride along by the same rows: recv_weight[slot[t,k]] = w[t,k]
        orw = oracle.dispatch_fp8(x_bits[:, :128], oslot, num_rows=R, topk_weights=w)[2] if w is not None else None
    if rw is not None:
        hw = host(rw)
        assert np.array_equal(hw[used], orw[used]) and np.all(hw[~used] == SENT_F32)


def routing(rng, T, K, E, distinct=True, mask_frac=0.0):
    if distinct and E >= K:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K]
    else:
        idx = rng.integers(0, E, size=(T, K))
    mask = rng.random((T, K)) < mask_frac
    bad = rng.choice(np.array([-1, E, E + 5, -7, 2 ** 31 - 1, -(2 ** 31)], dtype=np.int64), size=(T, K))
    return np.where(mask, bad, idx).astype(np.int32)


def tokens(rng, T, H, scale=1.0):
    return to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32) * np.float32(scale))


@pytest.mark.parametrize("cap", [0, 128, 5])
@pytest.mark.parametrize("fp8", [True, False])
def test_decode_workload(gpu, cap, fp8):
    wl = make_workload("decode", seed=3)
    print("case fused decode cap=%d fp8=%s" % (cap, fp8), flush=True)
    check_fused(gpu, wl.topk_idx, wl.x_bits, wl.topk_weights, wl.E, cap, fp8)


@pytest.mark.parametrize("T,K,E,H,cap,mask", [
    (1, 1, 1, 128, 0, 0.0),        # smallest
    (3, 2, 16, 256, 0, 0.3),       # masked ids
    (64, 3, 7, 384, 0, 0.1),       # generic K, odd E
    (37, 9, 300, 4224, 0, 0.05),   # generic K past one pass of 8 targets; 2nd chunk of 8 lanes
    (100, 16, 256, 1024, 3, 0.0),  # padded, heavy drops
    (32, 32, 64, 128, 0, 0.2),     # K at its maximum
    (384, 8, 256, 7168, 0, 0.0),   # exactly 3072 entries: one launch, 12 steps per lane
    (200, 8, 256, 2048, 9, 0.05),  # 1600 entries: 8 steps per lane, padded
    (96, 32, 1024, 128, 0, 0.0),   # E and K at their maximum with 3072 entries
])
def test_shapes(gpu, T, K, E, H, cap, mask):
    rng = np.random.default_rng(T * 7919 + K * 31 + E)
    idx = routing(rng, T, K, E, distinct=rng.random() < 0.5, mask_frac=mask)
    x = tokens(rng, T, H)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case fused T=%d K=%d E=%d H=%d cap=%d" % (T, K, E, H, cap), flush=True)
    check_fused(gpu, idx, x, w, E, cap, True)
    check_fused(gpu, idx, x, w, E, cap, False)


def test_all_entries_to_one_expert(gpu):
    """Every entry on expert 0, padded capacity below the count."""
    rng = np.random.default_rng(5)
    T, K, E, H = 200, 4, 64, 256
    idx = np.zeros((T, K), dtype=np.int32)
    x = tokens(rng, T, H)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case fused one expert", flush=True)
    check_fused(gpu, idx, x, w, E, 0, True)
    check_fused(gpu, idx, x, w, E, 100, True)


def test_every_entry_masked(gpu):
    rng = np.random.default_rng(6)
    T, K, E, H = 50, 8, 32, 128
    idx = np.full((T, K), -1, dtype=np.int32)
    x = tokens(rng, T, H)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case fused all masked", flush=True)
    check_fused(gpu, idx, x, w, E, 0, True)
    check_fused(gpu, idx, x, w, E, 4, False)


def test_empty_batch_writes_zero_counts(gpu):
    E = 256
    print("case fused T=0", flush=True)
    idx = np.zeros((0, 8), dtype=np.int32)
    x = np.zeros((0, 7168), dtype=np.uint16)
    check_fused(gpu, idx, x, None, E, 0, True)
    check_fused(gpu, idx, x, None, E, 16, True)


@pytest.mark.parametrize("T,K,cap", [(3073, 1, 0), (385, 8, 0), (512, 8, 0), (9000, 8, 0), (600, 8, 40)])
def test_fallback_paths(gpu, T, K, cap):
    """Past 3072 entries: the chunked kernel up to 65536 entries, beyond
    that the two-kernel layout (with the workspace) then the dispatch
    kernel."""
    rng = np.random.default_rng(T + K)
    E, H = 256, 512
    idx = routing(rng, T, K, E, distinct=True, mask_frac=0.05)
    x = tokens(rng, T, H, 20.0)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case fused fallback T=%d K=%d cap=%d" % (T, K, cap), flush=True)
    check_fused(gpu, idx, x, w, E, cap, True)


@pytest.mark.parametrize("seed", range(48))
def test_random(gpu, seed):
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.choice([1, 5, 64, 256, 1024]))
    K = int(rng.choice([1, 2, 4, 6, 8, 3, 13]))
    T = int(rng.choice([1, 17, 128, 255, 511]))
    T = min(T, 3072 // K)
    H = int(rng.choice([128, 1152, 2048, 7168]))
    cap = int(rng.choice([0, 0, 1, 8, 128]))
    if cap:
        cap = max(1, min(cap, 16_000_000 // (E * H)))  # padded buffers stay <= 32 MB
    idx = routing(rng, T, K, E, distinct=rng.random() < 0.6, mask_frac=float(rng.choice([0.0, 0.1])))
    x = tokens(rng, T, H, float(rng.choice([1e-3, 1.0, 100.0])))
    w = rng.standard_normal((T, K)).astype(np.float32)
    fp8 = bool(rng.random() < 0.7)
    print("case fused random seed=%d T=%d K=%d E=%d H=%d cap=%d fp8=%s" % (seed, T, K, E, H, cap, fp8), flush=True)
    check_fused(gpu, idx, x, w, E, cap, fp8, with_weight=bool(rng.random() < 0.5))


def test_convenience_calls_use_it(gpu):
    """ep.dispatch without a handle and ep.low_latency_dispatch go through
    the one call; their results equal the oracle's."""
    ep = gpu
    wl = make_workload("decode", seed=9)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(wl.topk_weights).cuda()
    print("case fused conveniences", flush=True)
    recv, scale, rw, h = ep.dispatch(x, idx, w, wl.E)
    oc, oo, oslot, osrc = oracle.dispatch_layout(wl.topk_idx, wl.E)
    assert np.array_equal(host(h.slot), oslot) and np.array_equal(host(h.expert_offset), oo)
    orecv, oscale, orw = oracle.dispatch_fp8(wl.x_bits, oslot, topk_weights=wl.topk_weights)
    nv = int(oo[-1])
    assert np.array_equal(host(recv)[:nv], orecv[:nv]) and np.array_equal(host(rw)[:nv], orw[:nv])
    r3, s3, cnt, ph = ep.low_latency_dispatch(x, idx, 128, wl.E)
    pc, pslot, psrc = oracle.dispatch_layout_padded(wl.topk_idx, wl.E, 128)
    assert np.array_equal(host(cnt), pc) and np.array_equal(host(ph.slot), pslot)
    precv, pscale, _ = oracle.dispatch_fp8(wl.x_bits, pslot, num_rows=wl.E * 128)
    used = (np.arange(128)[None, :] < pc[:, None]).ravel()
    assert np.array_equal(host(r3).reshape(-1, wl.H)[used], precv[used])
    assert np.array_equal(host(s3).reshape(-1, wl.H // 128)[used], pscale[used])
