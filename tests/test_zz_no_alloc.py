"""ep_layout_dispatch_noalloc (the allocation-free form of the one-call
layout + dispatch) against ep_layout_dispatch with a caller's workspace,
through the C ABI, bit for bit on every output.

Each case makes two calls in a row on one stream, the second with fewer
tokens, so the second reuses the library's scratch after the first has
filled it.  Shapes past 65536 entries take the two-launch layout, whose
per-chunk histograms live in that scratch; smaller shapes take the one-
launch kernels and touch no scratch.  Outputs start as sentinels, so rows
either call leaves untouched must match too.
"""

import numpy as np
import pytest
import torch

from tests.gpu_run import SENT_BF16, SENT_F32, SENT_I32, SENT_U8, to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu


def outputs(T, H, K, E, cap, fp8):
    R = E * cap if cap else T * K
    d = "cuda"
    o = {"counts": torch.full((E,), SENT_I32, dtype=torch.int32, device=d),
         "offsets": None if cap else torch.full((E + 1,), SENT_I32, dtype=torch.int32, device=d),
         "slot": torch.full((T, K), SENT_I32, dtype=torch.int32, device=d),
         "src": torch.full((R,), SENT_I32, dtype=torch.int32, device=d),
         "recv_weight": torch.full((R,), SENT_F32, dtype=torch.float32, device=d)}
    if fp8:
        o["recv"] = torch.full((R, H), SENT_U8, dtype=torch.uint8, device=d)
        o["scale"] = torch.full((R, H // 128), SENT_F32, dtype=torch.float32, device=d)
    else:
        o["recv"] = torch.full((R, H), SENT_BF16, dtype=torch.int16, device=d).view(torch.bfloat16)
        o["scale"] = None
    return o


def run(ep, wl, H, cap, fp8, noalloc):
    T, K, E = wl.T, wl.K, wl.E
    idx = to_dev(wl.topk_idx.astype(np.int32))
    w = to_dev(wl.topk_weights)
    x = to_dev(wl.x_bits[:, :H].copy().view(np.int16)).view(torch.bfloat16)
    o = outputs(T, H, K, E, cap, fp8)
    fmt = ep.EP_RECV_FP8_E4M3_G128 if fp8 else ep.EP_RECV_BF16
    args = (idx, x, w, E, cap, fmt, o["counts"], o["offsets"], o["slot"], o["src"], o["recv"], o["scale"],
            o["recv_weight"])
    if noalloc:
        ep.ep_layout_dispatch_noalloc(*args)
    else:
        nb = ep.ep_layout_workspace_bytes(T, K, E)
        ws = torch.full((max(nb, 16),), 0x5A, dtype=torch.uint8, device="cuda")
        ep.ep_layout_dispatch(*args, workspace=ws)
    torch.cuda.synchronize()
    return o


def same(a, b):
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k]), k


@pytest.mark.parametrize("name,T1,T2,H,cap,fp8", [
    ("prefill", 16384, 9000, 256, 0, True),     # 131072 then 72000 entries: scratch both times
    ("skew", 12000, 8500, 128, 0, False),       # BF16, skewed routing
    ("prefill", 10000, 8300, 128, 1024, True),  # padded layout past 65536 entries
    ("decode", 4096, 128, 256, 0, True),        # one-launch kernels, no scratch
])
def test_noalloc_matches_workspace_call(gpu, name, T1, T2, H, cap, fp8):
    ep = gpu
    for T in (T1, T2):
        wl = make_workload(name, seed=T, T=T)
        E, K = wl.E, wl.K
        need = ep.ep_layout_workspace_bytes(T, K, E)
        print("case noalloc %s T=%d H=%d cap=%d fp8=%d scratch=%d" % (name, T, H, cap, fp8, need), flush=True)
        assert need <= ep.EP_NOALLOC_SCRATCH_BYTES
        ref = run(ep, wl, H, cap, fp8, noalloc=False)
        got = run(ep, wl, H, cap, fp8, noalloc=True)
        same(got, ref)
