"""GPU parity of the low-latency (padded-capacity) layout and of dispatch /
combine driven by it, against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_F32, SENT_I32, SENT_U8, host, to_dev
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


def gpu_layout_padded(ep, idx, E, cap):
    T, K = idx.shape
    d_idx = to_dev(idx.astype(np.int32))
    count = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    slot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    src = torch.full((E * cap,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda") if nb else None
    ep.ep_dispatch_layout_padded(d_idx, E, cap, count, slot, src, ws)
    return count, slot, src


def check_layout(ep, idx, E, cap):
    count, slot, src = gpu_layout_padded(ep, idx, E, cap)
    oc, os_, osrc = oracle.dispatch_layout_padded(idx, E, cap)
    assert np.array_equal(host(count), oc)
    assert np.array_equal(host(slot), os_)
    used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
    hs = host(src)
    assert np.array_equal(hs[used], osrc[used])
    assert np.all(hs[~used] == SENT_I32)  # unused rows are not written
    return slot, os_


@pytest.mark.parametrize("name,T,cap", [("tiny", None, 64), ("tiny", None, 5), ("decode", None, 128),
                                        ("decode", None, 3), ("skew", 2048, 64), ("skew", 2048, 2048),
                                        ("prefill", None, 4096), ("hbm", 16384, 200)])
def test_padded_layout(gpu, name, T, cap):
    wl = make_workload(name, seed=0, T=T)
    print("case padded", name, wl.T, cap, flush=True)
    check_layout(gpu, wl.topk_idx, wl.E, cap)


@pytest.mark.parametrize("rows,E,cap", [(1024, 256, 7), (1025, 256, 9), (65536, 256, 300), (65537, 256, 100),
                                        (3000, 1024, 2), (70000, 1024, 64)])
def test_padded_layout_paths_and_masks(gpu, rows, E, cap):
    rng = np.random.default_rng(rows + cap)
    idx = rng.integers(-2, E + 1, size=(rows, 1)).astype(np.int32)
    print("case padded rows", rows, E, cap, flush=True)
    check_layout(gpu, idx, E, cap)


@pytest.mark.parametrize("name,cap", [("decode", 128), ("decode", 4), ("tiny", 3)])
def test_low_latency_pipeline(gpu, name, cap):
    """Padded layout -> FP8 dispatch into [E*cap, H] -> combine from
    [E*cap, H] expert outputs, bit-exact; dropped entries are skipped and
    unused rows stay untouched."""
    ep = gpu
    wl = make_workload(name, seed=1)
    T, H, E, K = wl.T, wl.H, wl.E, wl.K
    print("case low-latency pipeline", name, cap, flush=True)
    slot, oslot = check_layout(ep, wl.topk_idx, E, cap)
    R = E * cap
    d_x = to_dev(wl.x_bits.view(np.int16))
    d_w = to_dev(wl.topk_weights)
    recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
    scale = torch.full((R, H // 128), SENT_F32, dtype=torch.float32, device="cuda")
    rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(d_x, slot, d_w, ep.EP_RECV_FP8_E4M3_G128, recv, scale, rw, num_rows=R)
    orecv, oscale, orw = oracle.dispatch_fp8(wl.x_bits, oslot, num_rows=R, topk_weights=wl.topk_weights)
    used = np.zeros(R, bool)
    used[oslot[oslot >= 0]] = True
    hr, hs, hw = host(recv), host(scale), host(rw)
    assert np.array_equal(hr[used], orecv[used]) and np.all(hr[~used] == SENT_U8)
    assert np.array_equal(hs[used], oscale[used]) and np.all(hs[~used] == SENT_F32)
    assert np.array_equal(hw[used], orw[used])
    y = to_bf16_bits(np.random.default_rng(3).standard_normal((R, H), dtype=np.float32))
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(to_dev(y.view(np.int16)), slot, d_w, out, num_rows=R)
    assert np.array_equal(host(out), oracle.combine(y, oslot, wl.topk_weights))


def test_low_latency_wrappers(gpu):
    """The page-shaped wrappers: low_latency_dispatch returns [E, cap, H]
    rows and recv_expert_count; low_latency_combine reduces [E, cap, H]."""
    ep = gpu
    wl = make_workload("decode", seed=2)
    T, H, E = wl.T, wl.H, wl.E
    x = to_dev(wl.x_bits.view(np.int16))
    idx = torch.from_numpy(wl.topk_idx.astype(np.int64)).cuda()  # int64 ids are converted
    recv_x, recv_scale, count, h = ep.low_latency_dispatch(x, idx, T, E)
    oc, oslot, _ = oracle.dispatch_layout_padded(wl.topk_idx, E, T)
    assert tuple(recv_x.shape) == (E, T, H) and tuple(recv_scale.shape) == (E, T, H // 128)
    assert np.array_equal(host(count), oc)
    orecv, oscale, _ = oracle.dispatch_fp8(wl.x_bits, oslot, num_rows=E * T)
    hr = host(recv_x).reshape(E * T, H)
    for e in range(E):
        n = int(oc[e])
        assert np.array_equal(hr[e * T:e * T + n], orecv[e * T:e * T + n])
    y = torch.randn((E, T, H), device="cuda").to(torch.bfloat16)
    out = ep.low_latency_combine(y, h, torch.from_numpy(wl.topk_weights).cuda())
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16).reshape(E * T, H)
    assert np.array_equal(host(out.view(torch.int16)), oracle.combine(yb, oslot, wl.topk_weights))
