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


@pytest.mark.parametrize("capacity", [0, 128])
def test_step_plan_in_a_graph(gpu, capacity):
    """A plan built on a side stream and captured there: every replay, with
    new routing and tokens copied into the plan's inputs in between, equals
    the oracle for those inputs."""
    ep = gpu
    side = torch.cuda.Stream()
    wl = make_workload("decode", seed=21)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda()
    print("case plan graph", capacity, flush=True)
    plan = ep.StepPlan(idx, w, x, wl.E, capacity=capacity, stream=side)
    rng = np.random.default_rng(21)
    y = to_bf16_bits(rng.standard_normal((plan.rows, wl.H), dtype=np.float32))
    plan.y.copy_(torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        plan.step()  # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.step()
    for seed in (22, 23, 24):
        wl2 = make_workload("decode", seed=seed)
        idx.copy_(torch.from_numpy(wl2.topk_idx))
        w.copy_(torch.from_numpy(wl2.topk_weights))
        x.copy_(torch.from_numpy(wl2.x_bits.view(np.int16)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if capacity:
            oc, oslot, _ = oracle.dispatch_layout_padded(wl2.topk_idx, wl2.E, capacity)
            valid = (np.arange(capacity)[None, :] < oc[:, None]).ravel()
        else:
            oc, oo, oslot, _ = oracle.dispatch_layout(wl2.topk_idx, wl2.E)
            valid = np.arange(plan.rows) < oo[-1]
        assert np.array_equal(host(plan.counts), oc) and np.array_equal(host(plan.slot), oslot)
        orecv, oscale, _ = oracle.dispatch_fp8(wl2.x_bits, oslot, num_rows=plan.rows)
        assert np.array_equal(host(plan.recv_x)[valid], orecv[valid])
        assert np.array_equal(host(plan.recv_scale)[valid].view(np.uint32), oscale[valid].view(np.uint32))
        assert np.array_equal(host(plan.out.view(torch.int16)), oracle.combine(y, oslot, wl2.topk_weights))


def test_two_streams_at_once(gpu):
    """The library keeps no state: two plans stepping on two streams at the
    same time each produce their own oracle result."""
    ep = gpu
    plans, ys, wls = [], [], []
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print("case two streams", flush=True)
    for i, s in enumerate(streams):
        wl = make_workload("decode", seed=30 + i)
        idx = torch.from_numpy(wl.topk_idx).cuda()
        w = torch.from_numpy(wl.topk_weights).cuda()
        x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda()
        plan = ep.StepPlan(idx, w, x, wl.E, stream=s)
        y = to_bf16_bits(np.random.default_rng(30 + i).standard_normal((plan.rows, wl.H), dtype=np.float32))
        plan.y.copy_(torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16))
        plans.append(plan)
        ys.append(y)
        wls.append(wl)
    torch.cuda.synchronize()
    for _ in range(20):  # interleaved launches on the two streams
        for plan in plans:
            plan.step()
    torch.cuda.synchronize()
    for plan, y, wl in zip(plans, ys, wls):
        oc, oo, oslot, osrc = oracle.dispatch_layout(wl.topk_idx, wl.E)
        assert np.array_equal(host(plan.slot), oslot) and np.array_equal(host(plan.src), osrc)
        nv = int(oo[-1])
        orecv, oscale, _ = oracle.dispatch_fp8(wl.x_bits, oslot)
        assert np.array_equal(host(plan.recv_x)[:nv], orecv[:nv])
        assert np.array_equal(host(plan.out.view(torch.int16)), oracle.combine(y, oslot, wl.topk_weights))


def test_host_threads_at_once(gpu):
    """Four host threads step four plans at the same time, each on its own
    stream (ctypes releases the interpreter lock during every C call, so the
    library really is entered concurrently): packed, padded, a batch whose
    layout takes two launches through a workspace, and a tiny one.  Each
    plan's outputs match the oracle."""
    import threading

    ep = gpu
    # (workload, tokens, hidden, capacity); 9000 x 8 entries take the two-launch layout
    cases = [("decode", None, None, 0), ("decode", None, None, 64), ("skew", 9000, 256, 0), ("tiny", None, None, 0)]
    plans, ys, wls = [], [], []
    print("case host threads", flush=True)
    for i, (name, T, H, cap) in enumerate(cases):
        wl = make_workload(name, seed=40 + i, T=T, **({"H": H} if H else {}))
        idx = torch.from_numpy(wl.topk_idx).cuda()
        w = torch.from_numpy(wl.topk_weights).cuda()
        x = torch.from_numpy(wl.x_bits.view(np.int16)).cuda()
        plan = ep.StepPlan(idx, w, x, wl.E, capacity=cap, stream=torch.cuda.Stream())
        y = to_bf16_bits(np.random.default_rng(40 + i).standard_normal((plan.rows, wl.H), dtype=np.float32))
        plan.y.copy_(torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16))
        plans.append(plan)
        ys.append(y)
        wls.append(wl)
    torch.cuda.synchronize()
    errors = []

    def run(plan):
        try:
            for _ in range(25):
                plan.step()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(p,)) for p in plans]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for plan, y, wl, (name, T, H, cap) in zip(plans, ys, wls, cases):
        if cap:
            oc, oslot, osrc = oracle.dispatch_layout_padded(wl.topk_idx, wl.E, cap)
            valid = (oslot.ravel() >= 0)
            rows = np.unique(oslot.ravel()[valid])
        else:
            oc, oo, oslot, osrc = oracle.dispatch_layout(wl.topk_idx, wl.E)
            rows = np.arange(int(oo[-1]))
        assert np.array_equal(host(plan.counts), oc) and np.array_equal(host(plan.slot), oslot)
        orecv, oscale, _ = oracle.dispatch_fp8(wl.x_bits, oslot, num_rows=plan.rows)
        assert np.array_equal(host(plan.recv_x)[rows], orecv[rows])
        assert np.array_equal(host(plan.recv_scale)[rows].view(np.uint32), oscale[rows].view(np.uint32))
        assert np.array_equal(host(plan.out.view(torch.int16)), oracle.combine(y, oslot, wl.topk_weights))
