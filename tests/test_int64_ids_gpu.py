"""int64 expert ids (what routers usually produce) through the *_i64 entry
points, bit-exact against the oracle: every layout path, packed and
padded, the one-call dispatch, the conveniences and StepPlan.  Ids far
outside [0, E) must be masked, not truncated to 32 bits."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_I32, host, to_dev
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu

WIDE = np.array([2 ** 40, -(2 ** 33), -1, 2 ** 32 + 3, -(2 ** 40) + 5], dtype=np.int64)


def wide_ids(rng, T, K, E, frac=0.1):
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64) if E >= K else \
        rng.integers(0, E, size=(T, K)).astype(np.int64)
    mask = rng.random((T, K)) < frac
    idx = np.where(mask, rng.choice(np.concatenate([WIDE, [E, E + 2 ** 32]]), size=(T, K)), idx)
    return idx


def run_layout(ep, idx64, E, cap):
    T, K = idx64.shape
    d_idx = to_dev(idx64)
    assert d_idx.dtype == torch.int64
    R = E * cap if cap else T * K
    counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((R,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    if cap:
        ep.ep_dispatch_layout_padded(d_idx, E, cap, counts, slot, src, ws)
        return counts, None, slot, src
    offsets = torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_layout(d_idx, E, counts, offsets, slot, src, ws)
    return counts, offsets, slot, src


@pytest.mark.parametrize("T,K,E,cap", [(64, 8, 256, 0), (128, 8, 256, 0), (1000, 8, 256, 0), (9000, 8, 256, 0),
                                       (128, 8, 256, 16), (9000, 8, 256, 40), (300, 3, 1024, 0),
                                       (4096, 8, 1024, 0), (4096, 8, 512, 64)])
def test_layout_paths(gpu, T, K, E, cap):
    ep = gpu
    rng = np.random.default_rng(T + K + E + cap)
    idx = wide_ids(rng, T, K, E)
    print("case int64 layout T=%d K=%d E=%d cap=%d" % (T, K, E, cap), flush=True)
    counts, offsets, slot, src = run_layout(ep, idx, E, cap)
    if cap:
        oc, oslot, osrc = oracle.dispatch_layout_padded(idx, E, cap)
        used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
        assert np.array_equal(host(counts), oc) and np.array_equal(host(slot), oslot)
        assert np.array_equal(host(src)[used], osrc[used])
    else:
        oc, oo, oslot, osrc = oracle.dispatch_layout(idx, E)
        assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
        assert np.array_equal(host(slot), oslot) and np.array_equal(host(src), osrc)


@pytest.mark.parametrize("T,cap,fp8", [(128, 0, True), (128, 128, True), (128, 0, False), (384, 0, True),
                                       (600, 0, True), (64, 5, True)])
def test_one_call_dispatch(gpu, T, cap, fp8):
    """Decode kernel (up to 3072 entries) and the chunked kernel beyond."""
    ep = gpu
    E, K, H = 256, 8, 7168
    rng = np.random.default_rng(T + cap)
    idx = wide_ids(rng, T, K, E)
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    R = E * cap if cap else T * K
    print("case int64 one call T=%d cap=%d fp8=%s" % (T, cap, fp8), flush=True)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = None if cap else torch.empty(E + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    src = torch.empty(R, dtype=torch.int32, device="cuda")
    recv = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.int16, device="cuda")
    scale = torch.empty((R, H // 128), dtype=torch.float32, device="cuda") if fp8 else None
    rw = torch.empty(R, dtype=torch.float32, device="cuda")
    fmt = ep.EP_RECV_FP8_E4M3_G128 if fp8 else ep.EP_RECV_BF16
    ep.ep_layout_dispatch(to_dev(idx), to_dev(x.view(np.int16)), to_dev(w), E, cap, fmt, counts, offsets, slot, src,
                          recv, scale, rw)
    if cap:
        oc, oslot, _ = oracle.dispatch_layout_padded(idx, E, cap)
        used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
    else:
        oc, oo, oslot, _ = oracle.dispatch_layout(idx, E)
        used = np.arange(R) < oo[-1]
        assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(slot), oslot)
    orecv, oscale, orw = oracle.dispatch_fp8(x, oslot, num_rows=R, topk_weights=w)
    if fp8:
        assert np.array_equal(host(recv)[used], orecv[used])
        assert np.array_equal(host(scale)[used].view(np.uint32), oscale[used].view(np.uint32))
    else:
        assert np.array_equal(host(recv)[used], oracle.dispatch_bf16(x, oslot, num_rows=R)[used])
    assert np.array_equal(host(rw)[used], orw[used])


def test_conveniences_and_plan_keep_int64(gpu):
    """ep.dispatch / ep.low_latency_dispatch and StepPlan take int64 ids as
    they are (no narrowing cast) and match the oracle."""
    ep = gpu
    wl = make_workload("decode", seed=12)
    idx64 = wl.topk_idx.astype(np.int64)
    idx64[0, 0] = 2 ** 40  # masked, not truncated to expert 0
    d_idx = torch.from_numpy(idx64).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(wl.topk_weights).cuda()
    print("case int64 conveniences", flush=True)
    recv, scale, rw, h = ep.dispatch(x, d_idx, w, wl.E)
    oc, oo, oslot, osrc = oracle.dispatch_layout(idx64, wl.E)
    assert host(h.slot)[0, 0] == -1
    assert np.array_equal(host(h.slot), oslot) and np.array_equal(host(h.expert_offset), oo)
    r3, s3, cnt, ph = ep.low_latency_dispatch(x, d_idx, 128, wl.E)
    pc, pslot, _ = oracle.dispatch_layout_padded(idx64, wl.E, 128)
    assert np.array_equal(host(cnt), pc) and np.array_equal(host(ph.slot), pslot)
    plan = ep.StepPlan(d_idx, w, x, wl.E)
    y = to_bf16_bits(np.random.default_rng(12).standard_normal((plan.rows, wl.H), dtype=np.float32))
    plan.y.copy_(torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16))
    for separate in (False, True):
        if separate:
            plan.layout()
            plan.dispatch()
            plan.combine()
        else:
            plan.step()
        assert np.array_equal(host(plan.slot), oslot)
        assert np.array_equal(host(plan.out.view(torch.int16)), oracle.combine(y, oslot, wl.topk_weights))


@pytest.mark.parametrize("T,K,misalign", [(4096, 8, False), (4096, 8, True), (1001, 3, False), (1001, 3, True),
                                          (8191, 8, False)])
def test_one_launch_layout_id_loads(gpu, T, K, misalign):
    """The one-launch layout reads int64 ids two per 16-byte load when the ids
    are 16-byte aligned (odd T*K leaves a last id for the scalar tail), and
    one per load when they sit 8 bytes past a 16-byte boundary."""
    ep = gpu
    E = 256
    rng = np.random.default_rng(7 * T + K + misalign)
    idx = wide_ids(rng, T, K, E)
    print("case int64 one-launch layout T=%d K=%d misalign=%d" % (T, K, misalign), flush=True)
    n = T * K
    store = torch.empty(n + 2, dtype=torch.int64, device="cuda")
    d_idx = store[1:n + 1] if misalign else store[:n]
    d_idx.copy_(torch.from_numpy(idx.ravel()))
    d_idx = d_idx.view(T, K)
    assert (d_idx.data_ptr() % 16 == 8) == misalign
    counts = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((n,), SENT_I32, dtype=torch.int32, device="cuda")
    assert ep.ep_layout_workspace_bytes(T, K, E) == 0
    ep.ep_dispatch_layout(d_idx, E, counts, offsets, slot, src, None)
    oc, oo, oslot, osrc = oracle.dispatch_layout(idx, E)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), oslot) and np.array_equal(host(src), osrc)
