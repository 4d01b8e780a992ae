"""Pins for the oracle's backward helpers (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f32, combine, combine_backward, dispatch_backward, dispatch_layout, dot_rn32
from tests.pins import f32_mul, rn32, f32_frac
from tests.tolerances import grad_w_bound
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
    # the exact dot product rounded once: within half a binary32 ulp of the
    # float64 sum, whose own error is below H * 2^-53 * sum|g*y|
    terms = np.abs(bf16_bits_to_f32(g).astype(np.float64)[:, None, :] *
                   bf16_bits_to_f32(wl.y_bits).astype(np.float64)[np.where(slot >= 0, slot, 0)]).sum(-1)
    assert np.all(np.abs(gw - rw) <= 2.0 ** -24 * np.abs(rw) + 2.0 ** -38 * terms + 2.0 ** -149)
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


def test_combine_backward_exact_emulation():
    """Element-by-element: grad_y = BF16(RN32(w*g)), grad_w = RN32 of the
    exact rational sum of the products."""
    rng = np.random.default_rng(8)
    T, K, H = 3, 2, 48
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
                assert gw[t, k] == 0 and not np.signbit(gw[t, k])
                continue
            want_row = bf16(np.array([f32_mul(float(w[t, k]), float(v)) for v in gf[t]]))
            assert np.array_equal(gy[r], want_row)
            exact = sum((f32_frac(gf[t, c]) * f32_frac(yf[r, c]) for c in range(H)), f32_frac(0.0))
            assert float(gw[t, k]) == rn32(exact), (t, k)


def test_grad_w_is_rounded_once():
    """Sums where binary32 orders and the single rounding differ:
    [2^24, 1, 1, 1] is exactly 2^24 + 3, halfway between 2^24 + 2 and
    2^24 + 4, so it rounds to the even 2^24 + 4; adding in order keeps 2^24
    (every +1 is a tie to even) and pairwise gives 2^24 + 2.  And 1 + 2^-24
    + 2^-80: its nearest binary64 is the binary32 midpoint 1 + 2^-24, but
    the exact sum lies above it, so the answer is 1 + 2^-23, not 1."""
    a = np.array([2.0 ** 12, 1, 1, 1], np.float32)
    assert float(dot_rn32(a, a)) == 2.0 ** 24 + 4
    seq = np.float32(0)
    for v in a * a:
        seq = np.float32(seq + v)
    assert seq == 2.0 ** 24
    b = np.array([1.0, 2.0 ** -12, 2.0 ** -40], np.float32)
    assert float(dot_rn32(b, b)) == 1.0 + 2.0 ** -23
    assert float(dot_rn32(b[:2], b[:2])) == 1.0  # the exact tie goes to even
    assert float(dot_rn32(-b, b)) == -(1.0 + 2.0 ** -23)
    z = dot_rn32(np.array([1.0, -1.0], np.float32), np.array([1.0, 1.0], np.float32))
    assert z == 0 and not np.signbit(z)
    # the same values through combine_backward (one token, one pick)
    g = bf16(np.concatenate([a, np.zeros(4, np.float32)])[None, :])
    _, gw = combine_backward(g, g, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32))
    assert float(gw[0, 0]) == 2.0 ** 24 + 4


def test_grad_w_tolerance_covers_shallow_orders_and_catches_slips():
    """The GPU tolerance (tests/tolerances.py) against binary32 summation
    orders of the stated depth: 8-channel sums then a tree, 4-channel sums
    then a tree, on inputs with heavy cancellation, all inside the bound;
    a result with its largest product dropped, or with y taken from another
    row, falls outside it."""
    rng = np.random.default_rng(21)
    T, K, H = 64, 2, 7168
    scale = np.exp2(rng.integers(-6, 7, (T, H)))
    g = bf16(rng.standard_normal((T, H)) * scale)
    y = bf16(rng.standard_normal((T * K, H)) * np.exp2(rng.integers(-6, 7, (T * K, H))))
    slot = np.arange(T * K, dtype=np.int32).reshape(T, K)
    _, gw = combine_backward(g, y, slot, np.ones((T, K), np.float32))
    bound = grad_w_bound(g, y, slot)
    gf, yf = bf16_bits_to_f32(g), bf16_bits_to_f32(y)
    prod = (gf[:, None, :] * yf[slot]).astype(np.float32)  # exact
    for vec in (8, 4):
        part = np.zeros((T, K, H // vec), np.float32)
        for i in range(vec):
            part = (part + prod[:, :, i::vec]).astype(np.float32)
        while part.shape[-1] > 1:
            if part.shape[-1] % 2:
                part = np.concatenate([part, np.full(part.shape[:-1] + (1,), -0.0, np.float32)], -1)
            part = (part[..., 0::2] + part[..., 1::2]).astype(np.float32)
        assert np.all(np.abs(part[..., 0].astype(np.float64) - gw) <= bound), vec
    # the largest product dropped
    top = np.take_along_axis(prod, np.abs(prod).argmax(-1)[..., None], -1)[..., 0].astype(np.float64)
    assert np.all(np.abs((gw - top) - gw) > bound)
    _, gw_wrong = combine_backward(g, y, slot[:, ::-1].copy(), np.ones((T, K), np.float32))
    assert np.all(np.abs(gw_wrong.astype(np.float64) - gw) > bound)


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
