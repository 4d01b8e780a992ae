"""Pins for the oracle's backward helpers (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f32, combine, combine_backward, dispatch_backward, dispatch_layout,
                    pairwise_sum_f32)
from tests.pins import f32_add, f32_mul, rn32, f32_frac
from workloads import make_workload, to_bf16_bits


def bf16(a):
    return to_bf16_bits(np.asarray(a, dtype=np.float32))


def autograd_reference(g_bits, y_bits, slot, w):
    """float64 autograd of out[t] = sum_k w[t,k] * y[slot[t,k]] (masked k skipped)."""
    T, K = slot.shape
    y = torch.tensor(bf16_bits_to_f32(y_bits), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    mask = torch.tensor(slot >= 0)
    rows = torch.tensor(np.where(slot >= 0, slot, 0), dtype=torch.int64)
    out = (wt[:, :, None] * y[rows] * mask[:, :, None]).sum(dim=1)
    g = torch.tensor(bf16_bits_to_f32(g_bits), dtype=torch.float64)
    out.backward(g)
    return y.grad.numpy(), wt.grad.numpy()


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", 32)])
def test_combine_backward_matches_autograd(name, T):
    wl = make_workload(name, seed=4, T=T)
    _, _, slot, _ = dispatch_layout(wl.topk_idx, wl.E)
    slot = slot.copy()
    slot[1, 0] = -1  # a masked pick
    rng = np.random.default_rng(2)
    g = bf16(rng.standard_normal((wl.T, wl.H)))
    gy, gw = combine_backward(g, wl.y_bits, slot, wl.topk_weights)
    ry, rw = autograd_reference(g, wl.y_bits, slot, wl.topk_weights)
    used = np.zeros(gy.shape[0], bool)
    used[slot[slot >= 0]] = True
    gyf = bf16_bits_to_f32(gy[used]).astype(np.float64)
    # two roundings of one product: binary32 then BF16
    assert np.all(np.abs(gyf - ry[used]) <= np.abs(ry[used]) * (2.0 ** -8 + 2.0 ** -23) + 1e-38)
    # dot of H terms: 8 sequential adds + a tree of depth log2(H/8), each 2^-24
    terms = np.abs(bf16_bits_to_f32(g).astype(np.float64)[:, None, :] *
                   bf16_bits_to_f32(wl.y_bits).astype(np.float64)[np.where(slot >= 0, slot, 0)]).sum(-1)
    depth = 8 + int(np.ceil(np.log2(wl.H // 8))) + 1
    assert np.all(np.abs(gw - rw) <= depth * 2.0 ** -24 * terms + 1e-30)
    assert gw[1, 0] == 0 and np.signbit(gw[1, 0]) == 0


def test_dispatch_backward_matches_autograd():
    wl = make_workload("tiny", seed=5)
    _, _, slot, src = dispatch_layout(wl.topk_idx, wl.E)
    rng = np.random.default_rng(6)
    grec = bf16(rng.standard_normal((wl.T * wl.K, wl.H)))
    gx = dispatch_backward(grec, slot)
    # forward recv = x[src]; its adjoint scatters each row gradient back to its token
    x = torch.zeros((wl.T, wl.H), dtype=torch.float64, requires_grad=True)
    recv = x[torch.tensor(src.astype(np.int64))]
    recv.backward(torch.tensor(bf16_bits_to_f32(grec), dtype=torch.float64))
    ref = x.grad.numpy()
    got = bf16_bits_to_f32(gx).astype(np.float64)
    mag = np.abs(bf16_bits_to_f32(grec).astype(np.float64))[slot].sum(axis=1)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + wl.K * 2.0 ** -24 * mag + 1e-38)


def exact_pairwise(vals):
    """Recursive halving over a power-of-two padded list with explicit IEEE
    binary32 adds: an independent statement of the reduction tree."""
    n = 1
    while n < len(vals):
        n *= 2
    vals = list(vals) + [-0.0] * (n - len(vals))

    def rec(lo, hi):
        if hi - lo == 1:
            return vals[lo]
        mid = (lo + hi) // 2
        return f32_add(rec(lo, mid), rec(mid, hi))

    return rec(0, n)


def test_combine_backward_exact_emulation():
    """Element-by-element: grad_y = BF16(RN32(w*g)), grad_w by the stated order."""
    rng = np.random.default_rng(8)
    T, K, H = 3, 2, 48  # 6 vectors of 8 channels: the tree pads to 8 leaves
    g = bf16(rng.standard_normal((T, H)) * np.exp2(rng.integers(-20, 20, (T, 1))))
    y = bf16(rng.standard_normal((T * K, H)) * np.exp2(rng.integers(-20, 20, (T * K, 1))))
    w = (rng.standard_normal((T, K))).astype(np.float32)
    slot = np.array([[0, 3], [5, -1], [2, 4]], dtype=np.int32)
    gy, gw = combine_backward(g, y, slot, w)
    gf, yf = bf16_bits_to_f32(g), bf16_bits_to_f32(y)
    for t in range(T):
        for k in range(K):
            r = slot[t, k]
            if r < 0:
                assert gw[t, k] == 0
                continue
            want_row = bf16(np.array([f32_mul(float(w[t, k]), float(v)) for v in gf[t]]))
            assert np.array_equal(gy[r], want_row)
            parts = []
            for v in range(H // 8):
                acc = 0.0
                for c in range(8 * v, 8 * v + 8):
                    acc = f32_add(acc, f32_mul(float(gf[t, c]), float(yf[r, c])))
                parts.append(acc)
            assert float(gw[t, k]) == exact_pairwise(parts), (t, k)


def test_pairwise_tree_order_is_pinned():
    """A sum where the adjacent-pair tree and sequential order differ:
    [2^24, 1, 1, 1] gives (2^24 + 1 -> 2^24, a tie to even) + (1 + 1) =
    2^24 + 2 as a tree, but 2^24 sequentially (every +1 is a tie)."""
    v = np.array([[2.0 ** 24, 1.0, 1.0, 1.0]], np.float32)
    assert pairwise_sum_f32(v)[0] == 2.0 ** 24 + 2
    seq = np.float32(0)
    for x in v[0]:
        seq = np.float32(seq + x)
    assert seq == 2.0 ** 24
    assert exact_pairwise([2.0 ** 24, 1.0, 1.0, 1.0]) == 2.0 ** 24 + 2
    # -0.0 padding is an identity, including for signed zeros
    assert np.signbit(pairwise_sum_f32(np.array([[-0.0, -0.0, -0.0]], np.float32))[0])
    assert not np.signbit(pairwise_sum_f32(np.array([[0.0, -0.0, -0.0]], np.float32))[0])


def test_dispatch_backward_order_sensitive():
    """Copies summed in ascending k: [b, half a BF16 ulp of b, 0.375 ulp32,
    0.375 ulp32] keeps the exact tie (rounds to even); reversed order or
    exact summation rounds away."""
    rng = np.random.default_rng(13)
    T, K = 48, 4
    rows = []
    for _ in range(T):
        e = int(rng.integers(-20, 20))
        b = (1 + int(rng.integers(0, 64)) * 2 / 128) * 2.0 ** e
        small = 2.0 ** (e - 25) + 2.0 ** (e - 26)
        rows.append([b, 2.0 ** (e - 8), small, small])
    vals = np.array(rows, np.float32)
    grec = bf16(vals.reshape(-1, 1))
    assert np.array_equal(bf16_bits_to_f32(grec).reshape(T, K), vals)  # all exactly BF16
    slot = np.arange(T * K, dtype=np.int32).reshape(T, K)
    got = dispatch_backward(grec, slot)
    exact = bf16(vals.astype(np.float64).sum(axis=1).astype(np.float32)[:, None])
    assert np.all(got != exact)
    rev = dispatch_backward(grec, slot[:, ::-1].copy())
    assert np.all(rev != got)
    assert np.array_equal(got, combine(grec, slot, np.ones((T, K), np.float32)))
