"""GPU parity of the backward helpers against the oracle: the dispatch
backward and the row gradients bit-exact, the weight gradients (a dot
product over H channels, summed in the kernel's own order) within the
bound of tests/tolerances.py."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, gpu_layout, host, to_dev
from tests.tolerances import assert_grad_w_close, grad_w_bound
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


def rand_bf16(shape, seed):
    return to_bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


def run_backward(ep, idx, E, H, w, seed=0, with_w=True):
    T, K = idx.shape
    _, offsets, slot, _ = gpu_layout(ep, idx, E)
    oslot = oracle.dispatch_layout(idx, E)[2]
    R = T * K
    grec = rand_bf16((R, H), seed)
    y = rand_bf16((R, H), seed + 1)
    g = rand_bf16((T, H), seed + 2)
    # dispatch backward
    gx = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_dispatch_backward(to_dev(grec.view(np.int16)), slot, gx)
    assert np.array_equal(host(gx), oracle.dispatch_backward(grec, oslot))
    # combine backward
    gy = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
    gw = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda") if with_w else None
    ep.ep_combine_backward(to_dev(g.view(np.int16)), to_dev(y.view(np.int16)) if with_w else None, slot,
                           to_dev(w), gy, gw)
    ogy, ogw = oracle.combine_backward(g, y, oslot, w)
    used = np.zeros(R, bool)
    used[oslot[oslot >= 0]] = True
    hgy = host(gy)
    assert np.array_equal(hgy[used], ogy[used])
    assert np.all(hgy[~used] == SENT_BF16)
    if with_w:
        assert_grad_w_close(host(gw), ogw, grad_w_bound(g, y, oslot), oslot)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", None), ("skew", 1024)])
def test_backward_workloads(gpu, name, T):
    wl = make_workload(name, seed=3, T=T)
    print("case backward", name, wl.T, flush=True)
    run_backward(gpu, wl.topk_idx, wl.E, wl.H, wl.topk_weights, seed=5)


@pytest.mark.parametrize("H", [8, 72, 256, 384, 512, 520, 4096, 7168, 8192])
def test_backward_hidden_sizes(gpu, H):
    """H/8 vectors from 1 to 1024: tree padding inside a wave and across
    waves (1, 9, 32, 48, 64, 65, 512, 896, 1024 leaves)."""
    rng = np.random.default_rng(H)
    T, E, K = 37, 16, 4
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case backward H", H, flush=True)
    run_backward(gpu, idx, E, H, w, seed=H)


@pytest.mark.parametrize("K", [1, 3, 12])
def test_backward_runtime_k_and_masks(gpu, K):
    rng = np.random.default_rng(K)
    T, E, H = 50, 10, 256
    idx = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)  # masked ids and duplicates
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case backward K", K, flush=True)
    run_backward(gpu, idx, E, H, w, seed=K)
    run_backward(gpu, idx, E, H, w, seed=K, with_w=False)


def test_backward_wrappers(gpu):
    ep = gpu
    wl = make_workload("tiny", seed=9)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    h = ep.layout(idx, wl.E)
    R = wl.T * wl.K
    grec = torch.randn((R, wl.H), device="cuda").to(torch.bfloat16)
    y = torch.randn((R, wl.H), device="cuda").to(torch.bfloat16)
    g = torch.randn((wl.T, wl.H), device="cuda").to(torch.bfloat16)
    w = torch.from_numpy(wl.topk_weights).cuda()
    gx = ep.dispatch_backward(grec, h)
    gy, gw = ep.combine_backward(g, y, h, w)
    b = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    oslot = oracle.dispatch_layout(wl.topk_idx, wl.E)[2]
    assert np.array_equal(b(gx), oracle.dispatch_backward(b(grec), oslot))
    ogy, ogw = oracle.combine_backward(b(g), b(y), oslot, wl.topk_weights)
    assert np.array_equal(b(gy), ogy)
    assert_grad_w_close(gw.cpu().numpy(), ogw, grad_w_bound(b(g), b(y), oslot), oslot)
