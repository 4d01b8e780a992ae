"""The burst fan-out of BF16 token rows (from 16 MB of tokens): ep_dispatch
in BF16 and the row gradients of ep_combine_backward.  Each 1024-lane
workgroup (one per CU) loads up to 14 token vectors per lane and its
tokens' receive rows first, then writes the K copies.  Against the oracle,
bit-exact (the combine backward's weight gradients, a dot product in the
kernel's own order, within the bound of tests/tolerances.py); receive rows
no entry maps to keep their sentinel.

Cases: a last workgroup with fewer tokens, top-k through a runtime count
(10, 3), masked entries, the received routing weights, a small hidden size
with many tokens, and a batch split into several launches.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import SENT_BF16, SENT_F32, host, to_dev
from tests.tolerances import assert_grad_w_close, grad_w_bound
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def slots(rng, T, K, mask_frac):
    s = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    s[rng.random((T, K)) < mask_frac] = -1
    return s


@pytest.mark.parametrize("T,K,H,mask", [
    (4001, 8, 7168, 0.05),   # 16 tokens per workgroup, the last one holds one token
    (1200, 10, 7168, 0.0),   # runtime top-k
    (2100, 3, 4096, 0.1),    # odd top-k, 512 vectors per token
    (8192, 8, 1024, 0.02),   # 128 vectors per token, 32 tokens per workgroup
    (9000, 2, 7168, 0.0),    # three launches of 3000 tokens
])
@pytest.mark.parametrize("with_weight", [False, True])
def test_bf16_dispatch(gpu, T, K, H, mask, with_weight):
    ep = gpu
    assert T * H * 2 >= 16 << 20  # the burst path's size
    rng = np.random.default_rng(T + K + H)
    s = slots(rng, T, K, mask)
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    R = T * K
    print("case fan-out dispatch T=%d K=%d H=%d weight=%s" % (T, K, H, with_weight), flush=True)
    recv = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
    rw = torch.full((R,), SENT_F32, dtype=torch.float32, device="cuda") if with_weight else None
    ep.ep_dispatch(to_dev(x.view(np.int16)), to_dev(s), to_dev(w) if with_weight else None, ep.EP_RECV_BF16,
                   recv, None, rw)
    used = np.zeros(R, bool)
    used[s[s >= 0]] = True
    got = host(recv)
    assert np.array_equal(got[used], oracle.dispatch_bf16(x, s)[used])
    assert np.all(got[~used] == SENT_BF16)
    if with_weight:
        hw = host(rw)
        assert np.array_equal(hw[used], oracle.dispatch_fp8(x[:, :128], s, topk_weights=w)[2][used])
        assert np.all(hw[~used] == SENT_F32)


@pytest.mark.parametrize("T,K,H,mask", [(4001, 8, 7168, 0.05), (1500, 3, 7168, 0.1), (9000, 2, 7168, 0.0)])
def test_combine_backward_rows(gpu, T, K, H, mask):
    ep = gpu
    rng = np.random.default_rng(7 * T + K)
    s = slots(rng, T, K, mask)
    g = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    y = to_bf16_bits(rng.standard_normal((T * K, H), dtype=np.float32))
    w = rng.standard_normal((T, K)).astype(np.float32)
    R = T * K
    print("case fan-out combine backward T=%d K=%d" % (T, K), flush=True)
    gy = torch.full((R, H), SENT_BF16, dtype=torch.int16, device="cuda")
    gw = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    ep.ep_combine_backward(to_dev(g.view(np.int16)), to_dev(y.view(np.int16)), to_dev(s), to_dev(w), gy, gw)
    ogy, ogw = oracle.combine_backward(g, y, s, w)
    used = np.zeros(R, bool)
    used[s[s >= 0]] = True
    got = host(gy)
    assert np.array_equal(got[used], ogy[used])
    assert np.all(got[~used] == SENT_BF16)
    assert_grad_w_close(host(gw), ogw, grad_w_bound(g, y, s), s)
