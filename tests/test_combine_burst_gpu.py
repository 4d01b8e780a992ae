"""Combine of large batches (from 64 MB of gathered rows): each 1024-lane
workgroup (one per CU) holds up to 14 output vectors per lane and writes
them once their gathers are done; larger batches go as equal token slices,
one launch each.  Against the oracle, bit-exact, with the output rows of
other tokens untouched.

Cases: a last workgroup with fewer tokens (one token), top-k through the
generic loop (10) and small (2), a small hidden size with many tokens,
masked entries, unit weights (ep_dispatch_backward), and batches split
into several launches.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, host, to_dev
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def slots(rng, T, K, mask_frac):
    """Receive rows of (t, k): a random bijection onto T*K rows, with some
    entries masked (-1)."""
    s = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    s[rng.random((T, K)) < mask_frac] = -1
    return s


@pytest.mark.parametrize("T,K,H,mask", [
    (4001, 8, 7168, 0.05),   # 16 tokens per workgroup, the last one holds one token
    (500, 10, 7168, 0.0),    # generic top-k loop (8 + 2)
    (2400, 2, 7168, 0.1),    # K=2
    (4096, 8, 1024, 0.0),    # 128 work items per token: 2 per lane
    (3000, 8, 1536, 0.3),    # many masked entries
])
@pytest.mark.parametrize("unit", [False, True])
def test_burst_combine(gpu, T, K, H, mask, unit):
    ep = gpu
    assert T * K * H * 2 >= 64 << 20  # the burst path's size
    rng = np.random.default_rng(T + K + H)
    s = slots(rng, T, K, mask)
    y = to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case burst combine T=%d K=%d H=%d unit=%s" % (T, K, H, unit), flush=True)
    d_s = to_dev(s)
    d_y = to_dev(y.view(np.int16))
    out = torch.full((T + 1, H), SENT_BF16, dtype=torch.int16, device="cuda")  # one row past the output
    if unit:
        ep.ep_dispatch_backward(d_y, d_s, out[:T])
        want = oracle.dispatch_backward(y, s)
    else:
        ep.ep_combine(d_y, d_s, to_dev(w), out[:T])
        want = oracle.combine(y, s, w)
    got = host(out)
    assert np.array_equal(got[:T], want)
    assert np.all(got[T] == SENT_BF16)


@pytest.mark.parametrize("T,K,H", [(9000, 2, 7168), (8192, 8, 7168)])
def test_several_launches(gpu, T, K, H):
    """More tokens than 256 workgroups can hold at hidden 7168 (16 each):
    9000 tokens go as three launches of 3000 (12 tokens per workgroup),
    8192 as two of 4096."""
    ep = gpu
    rng = np.random.default_rng(T + K)
    s = slots(rng, T, K, 0.02)
    y = to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case burst combine launches T=%d K=%d" % (T, K), flush=True)
    out = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_combine(to_dev(y.view(np.int16)), to_dev(s), to_dev(w), out)
    assert np.array_equal(host(out), oracle.combine(y, s, w))


@pytest.mark.parametrize("T,K,H", [
    (131072, 32, 8),     # H = 8: one work item per token, a wavefront spans 64 tokens (T*K at its 2^22 limit)
    (64, 32, 16384),     # fewer tokens than CUs: one token per workgroup
    (37, 8, 114696),     # 14337 work items per token, more than a lane can hold: the per-item kernel
])
def test_extreme_shapes(gpu, T, K, H):
    ep = gpu
    assert T * K * H * 2 >= 64 << 20
    rng = np.random.default_rng(T + K + H)
    s = slots(rng, T, K, 0.05)
    y = to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    print("case burst combine extreme T=%d K=%d H=%d" % (T, K, H), flush=True)
    out = torch.full((T, H), SENT_BF16, dtype=torch.int16, device="cuda")
    ep.ep_combine(to_dev(y.view(np.int16)), to_dev(s), to_dev(w), out)
    assert np.array_equal(host(out), oracle.combine(y, s, w))
