"""StepPlan (pre-validated launches) against the oracle: packed and padded
layouts, FP8 and BF16 receive formats, every layout path, repeated steps."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_run import host
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("name,T,capacity,fp8", [("decode", None, 0, True), ("decode", None, 128, True),
                                                 ("decode", None, 0, False), ("tiny", None, 3, True),
                                                 ("skew", 9000, 0, True), ("prefill", None, 0, True)])
def test_step_plan_matches_oracle(gpu, name, T, capacity, fp8, separate):
    """separate: layout(), dispatch(), combine() as three calls instead of
    step() (layout and dispatch in one call, then combine)."""
    ep = gpu
    wl = make_workload(name, seed=7, T=T)
    print("case plan", name, wl.T, capacity, fp8, separate, flush=True)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda()
    plan = ep.StepPlan(idx, w, x, wl.E, capacity=capacity, fp8=fp8)
    rows = plan.rows
    rng = np.random.default_rng(7)
    y = to_bf16_bits(rng.standard_normal((rows, wl.H), dtype=np.float32))
    plan.y.copy_(torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16))
    for _ in range(2):  # the second step reuses every buffer
        if separate:
            plan.layout()
            plan.dispatch()
            plan.combine()
        else:
            plan.step()
    if capacity:
        oc, oslot, osrc = oracle.dispatch_layout_padded(wl.topk_idx, wl.E, capacity)
        assert np.array_equal(host(plan.counts), oc)
        used = (np.arange(capacity)[None, :] < oc[:, None]).ravel()
        assert np.array_equal(host(plan.src)[used], osrc[used])
        valid = used
    else:
        oc, oo, oslot, osrc = oracle.dispatch_layout(wl.topk_idx, wl.E)
        assert np.array_equal(host(plan.counts), oc) and np.array_equal(host(plan.offsets), oo)
        assert np.array_equal(host(plan.src), osrc)
        valid = np.arange(rows) < oo[-1]
    assert np.array_equal(host(plan.slot), oslot)
    if fp8:
        orecv, oscale, _ = oracle.dispatch_fp8(wl.x_bits, oslot, num_rows=rows)
        assert np.array_equal(host(plan.recv_x)[valid], orecv[valid])
        assert np.array_equal(host(plan.recv_scale)[valid].view(np.uint32), oscale[valid].view(np.uint32))
    else:
        orecv = oracle.dispatch_bf16(wl.x_bits, oslot, num_rows=rows)
        assert np.array_equal(host(plan.recv_x.view(torch.int16))[valid], orecv[valid])
    assert np.array_equal(host(plan.out.view(torch.int16)), oracle.combine(y, oslot, wl.topk_weights))
