"""Seeded random shapes (128 seeds) through every entry point against the
oracle: packed and padded layouts, FP8 and BF16 dispatch, combine, and
both backward helpers bit-exact, except combine_backward's weight
gradients (a dot product in the kernel's own order), which must lie
within the bound of tests/tolerances.py."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, SENT_F32, SENT_I32, SENT_U8, gpu_layout, host, to_dev
from tests.tolerances import assert_grad_w_close, grad_w_bound
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 3, 16, 64, 256, 300, 1024]))
    K = int(rng.choice([1, 2, 3, 4, 6, 8, 9, 16]))
    T = int(rng.choice([1, 5, 64, 127, 200, 513, 1500, 9000]))
    H = int(rng.choice([128, 256, 384, 1024, 2048, 7168]))
    if T * H > 2_000_000:
        T = max(1, 2_000_000 // H)
    if rng.random() < 0.5 and E >= K:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K]  # distinct experts
    else:
        idx = rng.integers(0, E, size=(T, K))  # duplicates allowed
    mask = rng.random((T, K)) < rng.choice([0.0, 0.05, 0.3])
    idx = np.where(mask, rng.choice([-1, E, -7]), idx).astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32) * np.float32(rng.choice([1e-3, 1.0, 50.0])))
    cap = int(rng.choice([1, 4, max(1, T // 4), T]))
    cap = max(1, min(cap, 16_000_000 // (E * H)))  # padded buffers stay <= 32 MB
    return T, H, E, K, idx, w, x, cap


@pytest.mark.parametrize("seed", range(128))
def test_random_shapes(gpu, seed):
    ep = gpu
    T, H, E, K, idx, w, x, cap = random_case(seed)
    print("case random seed=%d T=%d H=%d E=%d K=%d cap=%d" % (seed, T, H, E, K, cap), flush=True)
    d_w = to_dev(w)
    d_x = to_dev(x.view(np.int16))
    rng = np.random.default_rng(seed)

    # packed layout, FP8 dispatch, combine
    counts, offsets, slot, src = gpu_layout(ep, idx, E)
    oc, oo, os_, osrc = oracle.dispatch_layout(idx, E)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(slot), os_) and np.array_equal(host(src), osrc)
    R = T * K
    nv = int(oo[-1])
    recv = torch.full((R, H), SENT_U8, dtype=torch.uint8, device="cuda")
    scale = torch.full((R, H // 128), SENT_F32, dtype=torch.float32, device="cuda")
    rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(d_x, slot, d_w, ep.EP_RECV_FP8_E4M3_G128, recv, scale, rw)
    orecv, oscale, orw = oracle.dispatch_fp8(x, os_, topk_weights=w)
    assert np.array_equal(host(recv)[:nv], orecv[:nv])
    assert np.array_equal(host(scale)[:nv].view(np.uint32), oscale[:nv].view(np.uint32))
    assert np.array_equal(host(rw)[:nv], orw[:nv])
    y = to_bf16_bits(rng.standard_normal((R, H), dtype=np.float32))
    d_y = to_dev(y.view(np.int16))
    out = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_combine(d_y, slot, d_w, out)
    assert np.array_equal(host(out), oracle.combine(y, os_, w))

    # BF16 dispatch
    recv16 = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_dispatch(d_x, slot, None, ep.EP_RECV_BF16, recv16, None, None)
    assert np.array_equal(host(recv16)[:nv], oracle.dispatch_bf16(x, os_)[:nv])

    # backward helpers (H <= 8192 holds for every case)
    gx = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_dispatch_backward(d_y, slot, gx)
    assert np.array_equal(host(gx), oracle.dispatch_backward(y, os_))
    g = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    gy = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
    gw = torch.full((T, K), SENT_F32, dtype=torch.float32, device="cuda")
    ep.ep_combine_backward(to_dev(g.view(np.int16)), d_y, slot, d_w, gy, gw)
    ogy, ogw = oracle.combine_backward(g, y, os_, w)
    assert np.array_equal(host(gy)[:nv], ogy[:nv])
    assert_grad_w_close(host(gw), ogw, grad_w_bound(g, y, os_), os_)

    # padded layout and a dispatch / combine through it
    pc = torch.full((E,), SENT_I32, dtype=torch.int32, device="cuda")
    pslot = torch.full((T, K), SENT_I32, dtype=torch.int32, device="cuda")
    psrc = torch.full((E * cap,), SENT_I32, dtype=torch.int32, device="cuda")
    nb = ep.ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    ep.ep_dispatch_layout_padded(to_dev(idx), E, cap, pc, pslot, psrc, ws)
    opc, opslot, opsrc = oracle.dispatch_layout_padded(idx, E, cap)
    assert np.array_equal(host(pc), opc) and np.array_equal(host(pslot), opslot)
    used = (np.arange(cap)[None, :] < opc[:, None]).ravel()
    assert np.array_equal(host(psrc)[used], opsrc[used])
    PR = E * cap
    yp = to_bf16_bits(rng.standard_normal((PR, H), dtype=np.float32))
    outp = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_combine(to_dev(yp.view(np.int16)), pslot, d_w, outp, num_rows=PR)
    assert np.array_equal(host(outp), oracle.combine(yp, opslot, w))
