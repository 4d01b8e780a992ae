#!/usr/bin/env python3
"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

A step is one pass of the whole path over one batch: ep_layout_dispatch
(the layout and the FP8 E4M3 dispatch, one scale per 128 channels, in one
launch) -> ep_combine (BF16), on the prefill workload of the pages'
normal-kernel setting (4096 tokens, hidden 7168, 256 experts in 8 groups,
top-4 groups, top-8 experts).  The same step as three calls
(ep_dispatch_layout -> ep_dispatch -> ep_combine) is timed beside it.
Inputs are seeded synthetic tensors already resident in HBM when timing
starts.

    python bench.py [--steps K] [--warmup W]        # one JSON line
    python bench.py --workload hbm|skew|decode      # a JSON line for another configuration
    python bench.py --profile-pass [decode]         # short run for rocprofv3
    python bench.py --summarize-profile DIR         # rocprofv3 csv -> profiles/

The JSON line reports throughput as algorithmic bytes per second (bytes the
method must move, every one of the K copies counted), the per-kernel
launch durations (K back-to-back launches of each kernel between two HIP
events on the launch stream), the roofline of the dominant kernel (combine), p10 / median / p90 of single
steps warm and with the Infinity Cache flushed before each, the decode-size (128 tokens)
step time (eager launches through the checked binding and through
StepPlan, and as a replayed HIP graph, packed and with the low-latency
padded layout), the backward helpers at the prefill size, and
the oracle's CPU throughput on the same workload.
"""

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs and achieved HBM GB/s at 4096x7168 top-8; µs at 128 tok"
PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E peak
PROFILES = os.path.join(ROOT, "profiles")
# every kernel source: counter bytes are reported only while these are unchanged
KERNEL_SOURCES = sorted("combine_ep_dispatch_amd/csrc/" + f for f in os.listdir(os.path.join(ROOT, "combine_ep_dispatch_amd", "csrc"))
                        if f.endswith((".hip", ".h")))
TRAFFIC_FILE = os.path.join(PROFILES, "prefill_4096x7168_top8_counter_traffic.txt")
# the prefill step's kernels as they appear in the profile, and the separate
# layout and dispatch kernels of the three-call form, timed beside them
STEP_KERNELS = {"layout_dispatch": "layout_dispatch_split<true, int, true, true, true, 7>",
                "combine": "combine_burst_kernel<8, false>"}
REF_KERNELS = {"layout": "layout_fused<16, true, int>", "dispatch": "dispatch_fp8_kernel<8, true, true>"}
PROFILED_KERNELS = dict(STEP_KERNELS, **REF_KERNELS)


def backward_bytes(T, H, K):
    """Algorithmic bytes of the backward helpers: dispatch_backward reads the
    K row gradients and writes the token gradient; combine_backward reads
    grad_out and the K expert rows and writes K row gradients and K weights."""
    dispatch_bwd = 2 * T * K * H + 4 * T * K + 2 * T * H
    combine_bwd = 2 * T * H + 2 * T * K * H + 8 * T * K + 2 * T * K * H + 4 * T * K
    return dispatch_bwd, combine_bwd


def alg_bytes(T, H, E, K, fp8=True):
    """Bytes each kernel must move (reads + writes), all K copies counted."""
    layout = 12 * T * K + 8 * E + 4  # idx in; slot, src out; counts, offsets out
    if fp8:
        dispatch = 2 * T * H + 4 * T * K + T * K * H + 4 * T * K * (H // 128)
    else:
        dispatch = 2 * T * H + 4 * T * K + 2 * T * K * H
    combine = 2 * T * K * H + 8 * T * K + 2 * T * H
    return layout, dispatch, combine


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Setup:
    """Device buffers of one workload plus closures for the three calls."""

    def __init__(self, ep, torch, name, seed=0, capacity=0):
        """capacity > 0: the low-latency layout with that many rows per
        expert (receive and expert-output buffers of E*capacity rows)."""
        from workloads import make_workload

        wl = make_workload(name, seed=seed)
        self.wl = wl
        T, H, E, K = wl.T, wl.H, wl.E, wl.K
        self.capacity = capacity
        R = E * capacity if capacity else T * K
        self.rows = R
        dev = "cuda"
        self.idx = torch.from_numpy(wl.topk_idx).to(dev)
        self.w = torch.from_numpy(wl.topk_weights).to(dev)
        self.x = torch.from_numpy(wl.x_bits.view("int16")).to(dev)
        # expert outputs for combine: the workload's own N(0,1) BF16 rows (the
        # CPU baseline combines the same ones); the padded layout's E*capacity
        # rows are drawn on the device instead
        if wl.fp8:
            if capacity:
                g = torch.Generator(device=dev)
                g.manual_seed(1000 + seed)
                self.y = torch.randn((R, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            else:
                self.y = torch.from_numpy(wl.y_bits.view("int16")).to(dev).view(torch.bfloat16)
            self.recv = torch.empty((R, H), dtype=torch.uint8, device=dev)
            self.scale = torch.empty((R, H // 128), dtype=torch.float32, device=dev)
            self.fmt = ep.EP_RECV_FP8_E4M3_G128
        else:
            self.recv = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
            self.scale = None
            self.y = self.recv  # identity expert: combine reads the receive buffer
            self.fmt = ep.EP_RECV_BF16
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.slot = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.src = torch.empty(R if capacity else T * K, dtype=torch.int32, device=dev)
        nb = ep.ep_layout_workspace_bytes(T, K, E)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.ep = ep
        self.bytes = alg_bytes(T, H, E, K, wl.fp8)

    def layout(self):
        if self.capacity:
            self.ep.ep_dispatch_layout_padded(self.idx, self.wl.E, self.capacity, self.counts, self.slot, self.src,
                                              self.ws)
        else:
            self.ep.ep_dispatch_layout(self.idx, self.wl.E, self.counts, self.offsets, self.slot, self.src, self.ws)

    def dispatch(self):
        self.ep.ep_dispatch(self.x, self.slot, None, self.fmt, self.recv, self.scale, None, num_rows=self.rows)

    def combine(self):
        self.ep.ep_combine(self.y, self.slot, self.w, self.out, num_rows=self.rows)

    def step(self):
        """The three-call form: layout, dispatch, combine."""
        self.layout()
        self.dispatch()
        self.combine()

    def bare(self):
        """A StepPlan on the same inputs: the same kernels, launched through
        pre-built C calls, so back-to-back launches of a short kernel are
        not paced by the host."""
        if getattr(self, "_plan", None) is None:
            self._plan = self.ep.StepPlan(self.idx, self.w, self.x, self.wl.E, capacity=self.capacity,
                                          fp8=self.wl.fp8, y=self.y)
        return self._plan

    def layout_dispatch(self):
        # one call for layout + dispatch (one launch up to 65536 entries)
        self.ep.ep_layout_dispatch(self.idx, self.x, None, self.wl.E, self.capacity, self.fmt, self.counts,
                                   None if self.capacity else self.offsets, self.slot, self.src, self.recv,
                                   self.scale, None, self.ws)

    def step_fused(self):
        """Layout and dispatch in one call, then combine."""
        self.layout_dispatch()
        self.combine()

    def backward_buffers(self, torch):
        T, H, K = self.wl.T, self.wl.H, self.wl.K
        self.grad_out = torch.randn((T, H), device="cuda").to(torch.bfloat16)
        self.grad_x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        self.grad_y = torch.empty((self.rows, H), dtype=torch.bfloat16, device="cuda")
        self.grad_w = torch.empty((T, K), dtype=torch.float32, device="cuda")

    def dispatch_backward(self):
        # the expert-output tensor stands in for the receive-row gradients
        self.ep.ep_dispatch_backward(self.y, self.slot, self.grad_x, num_rows=self.rows)

    def combine_backward(self):
        self.ep.ep_combine_backward(self.grad_out, self.y, self.slot, self.w, self.grad_y, self.grad_w,
                                    num_rows=self.rows)


def time_steps(torch, s, steps, warmup, fused=False):
    """K steps bracketed by synchronisation, timed with HIP events on the
    stream the kernels are launched on; then, for each call, K back-to-back
    launches of it (bare C calls on the same inputs) between two events:
    its mean launch duration, the kernel plus one launch gap.  An event
    recorded between every two calls would add ~5 µs to each interval on
    MI355X.  fused: the step is ep_layout_dispatch + ep_combine, and the
    separate layout and dispatch kernels are timed too; else the three
    calls."""
    stream = torch.cuda.current_stream()
    step = s.step_fused if fused else s.step
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us_step = a.elapsed_time(b) * 1e3 / steps
    plan = s.bare()
    plan.layout()
    calls = [("layout", plan.layout), ("dispatch", plan.dispatch), ("combine", plan.combine)]
    if fused:
        calls = [("layout_dispatch", plan.layout_dispatch)] + calls
    per = {name: time_loop(torch, fn, steps, 1) for name, fn in calls}
    return us_step, per, wall


def step_times(torch, step, reps, flush_bytes=0, warmup=3):
    """Durations (µs) of `reps` steps, each timed on its own with one HIP
    event before and one after it on the launch stream (no event between
    the step's calls: an event there adds a few µs to what follows it).
    flush_bytes > 0: before every step, outside its events, a device read of
    that many bytes (a reduction) evicts the 256 MB Infinity Cache, so the
    step starts from HBM.  A write fill would evict it too, but leaves that
    many dirty lines whose write-back then slows the next kernel (measured:
    the dispatch kernel 66 µs instead of 54)."""
    stream = torch.cuda.current_stream()
    scratch = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda") if flush_bytes else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = []
    for _ in range(reps):
        if scratch is not None:
            scratch.max()
        m = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        m[0].record(stream)
        step()
        m[1].record(stream)
        marks.append(m)
    torch.cuda.synchronize()
    del scratch
    return [m[0].elapsed_time(m[1]) * 1e3 for m in marks]


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def dist(v):
    return {"p10": round(pct(v, 0.1), 2), "median": round(pct(v, 0.5), 2), "p90": round(pct(v, 0.9), 2)}


FLUSH_BYTES = 512 << 20


def time_loop(torch, fn, steps, warmup):
    """Mean µs of fn over `steps` back-to-back calls, HIP events only at the
    ends (on the launch stream)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


def time_graph(torch, step, replays, steps_per_graph=1):
    """`step` captured `steps_per_graph` times in one HIP graph and replayed;
    returns µs per step (events on the stream the graph is launched on)."""
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps_per_graph):
            step()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * steps_per_graph)


def host_submit_us(torch, step, n):
    """Host time per call of `step` over n calls issued back to back (no
    synchronisation inside the loop): when it reaches the GPU time per
    step, eager timing measures the launches' host cost, not the kernels."""
    import time
    for _ in range(10):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return (t1 - t0) / n * 1e6


def read_traffic():
    """HBM bytes per launch of the profiled prefill kernels (the keys of
    PROFILED_KERNELS) from the committed rocprofv3 counter summary, or None
    when any kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_hash(KERNEL_SOURCES):
        return None
    try:
        return {step: float(vals["hbm_bytes_per_launch[%s]" % step]) for step in PROFILED_KERNELS}
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s):
    """The oracle, untuned, on the same arrays the GPU step uses: the layout
    of all T*K entries, then, 512 tokens at a time, FP8 dispatch of those
    tokens into their real receive rows (the layout's slots) and combine of
    those tokens from the workload's expert outputs y gathered through the
    same slots.  Whole passes repeat until the time budget is spent; numpy
    runs these ops on one thread."""
    import numpy as np  # noqa: F401

    import oracle

    T, H, E, K = wl.T, wl.H, wl.E, wl.K
    step_b = sum(alg_bytes(T, H, E, K, True))
    chunk = 512
    x, y, w = wl.x_bits, wl.y_bits, wl.topk_weights
    R = T * K
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < budget_s:
        _, _, slot, _ = oracle.dispatch_layout(wl.topk_idx, E)
        for t in range(0, T, chunk):
            oracle.dispatch_fp8(x[t:t + chunk], slot[t:t + chunk], num_rows=R)
            oracle.combine(y, slot[t:t + chunk], w[t:t + chunk])
        passes += 1
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(passes * step_b / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": "%d full pass(es) over the prefill workload's own arrays (4096 tokens x 7168, top-8, "
                      "seed 0): layout of all 32768 entries, then FP8 dispatch into the real receive rows and "
                      "combine of the same expert outputs y the GPU combines, gathered through the real slots, "
                      "512 tokens at a time; %.1f s, numpy single-threaded; %d host CPUs visible"
                      % (passes, dt, os.cpu_count())}


def profile_pass(ep, torch, workload="prefill"):
    """Short run for rocprofv3: a plain 1 GiB device copy (counter
    calibration: known bytes read and written), then 5 steps of the
    workload (prefill by default): three calls, then layout and dispatch in
    one call."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    s = Setup(ep, torch, workload, 0)
    for _ in range(5):
        s.step()
    for _ in range(5):
        s.step_fused()
    if workload == "prefill":
        s.backward_buffers(torch)
        for _ in range(3):
            s.dispatch_backward()
            s.combine_backward()
    torch.cuda.synchronize()
    print("profile pass done", flush=True)


PROFILE_COMMANDS = """\
(from the repository root; OUT is any scratch directory; run rocprofv3 with TMPDIR=/tmp)
rocprofv3 --kernel-trace --stats -d OUT/prof_trace -o trace --output-format csv -- python3 bench.py --profile-pass
rocprofv3 --pmc FETCH_SIZE -d OUT/prof_fetch -o fetch --output-format csv -- python3 bench.py --profile-pass
rocprofv3 --pmc WRITE_SIZE -d OUT/prof_write -o write --output-format csv -- python3 bench.py --profile-pass
rocprofv3 --kernel-trace --stats -d OUT/prof_decode -o decode --output-format csv -- python3 bench.py --profile-pass decode
rocprofv3 --kernel-trace --stats -d OUT/prof_hbm_trace -o trace --output-format csv -- python3 bench.py --profile-pass hbm
rocprofv3 --pmc FETCH_SIZE -d OUT/prof_hbm_fetch -o fetch --output-format csv -- python3 bench.py --profile-pass hbm
rocprofv3 --pmc WRITE_SIZE -d OUT/prof_hbm_write -o write --output-format csv -- python3 bench.py --profile-pass hbm
rocprofv3 --kernel-trace --stats -d OUT/prof_bench -o bench --output-format csv -- python3 bench.py > OUT/bench_under_rocprof.json
python3 bench.py --summarize-profile OUT
"""

COPY_BYTES = 1 << 30  # the profile pass's plain device copy


def summarize_profile(dirname):
    """rocprofv3 csv output (three runs, see PROFILE_COMMANDS) -> short text
    summaries under profiles/.  Counters are KiB per dispatch; each is scaled
    by what it reads for the plain 1 GiB copy (bytes known exactly)."""
    import csv

    def rows(sub, pattern):
        out = []
        for f in sorted(glob.glob(os.path.join(dirname, sub, "**", pattern), recursive=True)):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("ep::", "")
        return name.split("(")[0]

    stats = rows("prof_trace", "*kernel_stats.csv")
    lines = ["rocprofv3 kernel trace: prefill workload (4096 tokens, hidden 7168, 256 experts, top-8,",
             "FP8 dispatch, BF16 combine), 5 steps after a 1 GiB device copy", "", "commands:", PROFILE_COMMANDS,
             "%-40s %6s %12s %12s %12s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns")]
    for r in stats:
        lines.append("%-40s %6s %12.0f %12.0f %12.0f" % (short(r["Name"])[:40], r["Calls"], float(r["AverageNs"]),
                                                         float(r["MinNs"]), float(r["MaxNs"])))
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "prefill_4096x7168_top8_kernel_trace.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    dec = rows("prof_decode", "*kernel_trace.csv")
    if dec:
        # steady state: the last 3 of 5 three-call steps (layout, dispatch,
        # combine), then the last 3 of 5 fused steps (layout_dispatch, combine)
        fwd = ("layout", "dispatch_fp8_kernel", "combine_kernel<8, false,")
        ours = [r for r in dec if short(r["Kernel_Name"]).startswith(fwd)]
        three = ours[:15][-9:]
        fused = ours[15:][-6:]
        lines = ["rocprofv3 kernel trace: decode workload (128 tokens, hidden 7168, 256 experts, top-8,",
                 "FP8 dispatch, BF16 combine): last 3 of 5 eager three-call steps, then last 3 of 5 eager",
                 "fused steps (layout and dispatch in one launch)", "", "commands:", PROFILE_COMMANDS,
                 "%-40s %10s" % ("kernel", "dur_ns")]
        for r in three + [None] + fused:
            if r is None:
                lines.append("")
                continue
            lines.append("%-40s %10d" % (short(r["Kernel_Name"])[:40],
                                         int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        with open(os.path.join(PROFILES, "decode_128x7168_top8_kernel_trace.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")

    def counters(fetch_sub, write_sub):
        """{kernel: bytes per launch} from the two counter runs, and the
        calibration lines (each counter scaled by what it reads for the
        profile pass's plain 1 GiB device copy)."""
        agg = {}
        for sub in (fetch_sub, write_sub):
            for r in rows(sub, "*counter_collection.csv"):
                agg.setdefault((short(r["Kernel_Name"]), r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        avg = {k: sum(v) / len(v) for k, v in agg.items()}
        copy_kib = COPY_BYTES / 1024.0
        cf, cw = avg[("__amd_rocclr_copyBuffer", "FETCH_SIZE")], avg[("__amd_rocclr_copyBuffer", "WRITE_SIZE")]
        f_fetch, f_write = copy_kib / cf, copy_kib / cw
        cal = ["calibration: plain 1 GiB device copy (__amd_rocclr_copyBuffer) reads FETCH_SIZE %.1f KiB and "
               "WRITE_SIZE %.1f KiB" % (cf, cw), "fetch_scale: %.4f" % f_fetch, "write_scale: %.4f" % f_write]
        per = {}
        for kern in {k for (k, c) in avg}:
            fk, wk = avg.get((kern, "FETCH_SIZE")), avg.get((kern, "WRITE_SIZE"))
            if fk is not None and wk is not None:
                per[kern] = (fk * 1024 * f_fetch, wk * 1024 * f_write)
        return per, cal

    def traffic_lines(per, known):
        out = []
        for prefix, a in known:
            for kern in sorted(k for k in per if k.startswith(prefix)):
                fb, wb = per[kern]
                out.append("%-58s fetch %12.0f B  write %12.0f B  total %12.0f B  algorithmic %12d B  ratio %.4f"
                           % (kern, fb, wb, fb + wb, a, (fb + wb) / a))
        return out

    per, cal = counters("prof_fetch", "prof_write")
    T, H, E, K = 4096, 7168, 256, 8
    alg = dict(zip(("layout", "dispatch_fp8_kernel", "combine_kernel"), alg_bytes(T, H, E, K, True)))
    alg["layout_dispatch_split"] = alg["layout"] + alg["dispatch_fp8_kernel"]
    lines = ["HBM traffic per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (two separate --pmc runs),",
             "prefill workload (4096 x 7168, 256 experts, top-8, FP8 dispatch, BF16 combine).", "",
             "commands:", PROFILE_COMMANDS] + cal + [""]
    d_bwd, _ = backward_bytes(T, H, K)
    known = (("layout_fused", alg["layout"]),
             ("layout_dispatch_split", alg["layout_dispatch_split"]),
             ("dispatch_fp8_kernel", alg["dispatch_fp8_kernel"]),
             ("combine_kernel<8, false,", alg["combine_kernel"]),
             ("combine_burst_kernel<8, false>", alg["combine_kernel"]),
             ("combine_kernel<8, true,", d_bwd),  # ep_dispatch_backward
             ("combine_burst_kernel<8, true>", d_bwd),
             ("grad_rows_kernel", 2 * T * H + 8 * T * K + 2 * T * K * H),
             ("fanout_burst_bf16<true", 2 * T * H + 8 * T * K + 2 * T * K * H),  # the same, as a burst
             ("grad_weights_kernel", 2 * T * H + 2 * T * K * H + 8 * T * K))
    lines += traffic_lines(per, known)
    totals = {k: f + w for k, (f, w) in per.items()}
    lines += ["", "the prefill step's kernels (combine is the roofline's dominant kernel), then the separate",
              "layout and dispatch kernels of the three-call form:"]
    lines += ["hbm_bytes_per_launch[%s]: %.0f" % (step, totals[kern]) for step, kern in PROFILED_KERNELS.items()]
    lines += ["source_sha256: %s" % source_hash(KERNEL_SOURCES),
              "(sha256 prefix of every file under combine_ep_dispatch_amd/csrc; bench.py reports counter bytes "
              "only while it matches)"]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    written = ["prefill_4096x7168_top8_kernel_trace.txt", "decode_128x7168_top8_kernel_trace.txt",
               os.path.basename(TRAFFIC_FILE)]
    if rows("prof_hbm_fetch", "*counter_collection.csv"):
        written.append(summarize_hbm(dirname, rows, short, counters, traffic_lines))
    if summarize_bench_run(dirname, rows, short):
        written.append(BENCH_RUN_FILE)
    for p in written:
        if os.path.exists(os.path.join(PROFILES, p)):
            print(open(os.path.join(PROFILES, p)).read())


BENCH_RUN_FILE = "prefill_4096x7168_top8_bench_run.txt"
HBM_FILE = "hbm_32768x7168_top8_bf16_counter_traffic.txt"


def summarize_hbm(dirname, rows, short, counters, traffic_lines):
    """The 32768-token BF16 workload: kernel durations (trace) and HBM bytes
    per launch (counters) of its layout kernels, its burst fan-out (8
    launches of 4096 tokens each) and its burst combine (likewise)."""
    T, H, E, K = 32768, 7168, 256, 8
    lay, dis, com = alg_bytes(T, H, E, K, fp8=False)
    slice_t = 4096
    dis_launch = alg_bytes(slice_t, H, E, K, fp8=False)[1]
    com_launch = alg_bytes(slice_t, H, E, K, fp8=False)[2]
    per, cal = counters("prof_hbm_fetch", "prof_hbm_write")
    stats = {short(r["Name"]): r for r in rows("prof_hbm_trace", "*kernel_stats.csv")}
    lines = ["32768-token BF16 workload (32768 x 7168, 256 experts, top-8, BF16 dispatch into a 3.76 GB receive",
             "buffer, BF16 combine of that buffer): rocprofv3 kernel durations and HBM bytes per launch from",
             "FETCH_SIZE and WRITE_SIZE (separate --pmc runs), 5 three-call steps then 5 one-call steps after a",
             "1 GiB device copy.  The layout is two kernels (layout_count, layout_finalize: 12TK + 8E + 4 B in",
             "all); the BF16 dispatch and the combine each run as 8 launches of 4096 tokens (algorithmic bytes",
             "per launch: dispatch 2*4096*H + 4*4096*K + 2*4096*K*H, combine 2*4096*K*H + 8*4096*K + 2*4096*H).",
             "", "commands:", PROFILE_COMMANDS] + cal + ["",
             "%-58s %6s %12s %14s" % ("kernel", "calls", "avg_us", "alg_GBs/launch")]
    per_launch = {"layout_count": None, "layout_finalize": None, "fanout_burst_bf16<false": dis_launch,
                  "combine_burst_kernel<8, false>": com_launch}
    for name, r in sorted(stats.items()):
        a = next((v for k, v in per_launch.items() if name.startswith(k)), None)
        us = float(r["AverageNs"]) / 1e3
        lines.append("%-58s %6s %12.2f %14s" % (name[:58], r["Calls"], us,
                                                "%.1f" % (a / us / 1e3) if a else "-"))
    lines += ["", "HBM bytes per launch:"]
    lines += traffic_lines(per, (("layout_count", lay), ("layout_finalize", lay),
                                 ("fanout_burst_bf16<false", dis_launch),
                                 ("combine_burst_kernel<8, false>", com_launch)))
    lines += ["(the layout kernels' ratios compare each launch with the whole layout's algorithmic bytes)",
              "source_sha256: %s" % source_hash(KERNEL_SOURCES)]
    with open(os.path.join(PROFILES, HBM_FILE), "w") as f:
        f.write("\n".join(lines) + "\n")
    return HBM_FILE


def summarize_bench_run(dirname, rows, short):
    """The default bench command run under rocprofv3 --kernel-trace: the
    profiler's mean duration of each prefill step kernel over all its
    launches in that process, beside the HIP-event durations (kernel_us)
    that the same process printed in its JSON line."""
    stats = {short(r["Name"]): r for r in rows("prof_bench", "*kernel_stats.csv")}
    trace = rows("prof_bench", "*kernel_trace.csv")
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    path = os.path.join(dirname, "bench_under_rocprof.json")
    if not stats or not os.path.exists(path):
        return False
    rec = None
    for line in open(path):
        if line.startswith("{"):
            rec = json.loads(line)
    if rec is None:
        return False
    def b2b_run(kern, at_least):
        """Durations of the first run of at least `at_least` consecutive
        launches of `kern` with no other kernel between them: the prefill
        back-to-back loop that kernel_us times (the same kernel also runs
        inside steps, after another kernel, where its mean differs, and
        later in the run for other workloads)."""
        cur = []
        for r in trace + [None]:
            if r is not None and short(r["Kernel_Name"]) == kern:
                cur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                continue
            if len(cur) >= at_least:
                return cur
            cur = []
        return []

    lines = ["The default bench command under rocprofv3 --kernel-trace --stats.  For each prefill step kernel:",
             "the profiler's mean duration over all its launches in the process (timed steps, back-to-back",
             "loops, single-step timings, warm and flushed, graph replays), and its mean over the launches of",
             "the back-to-back loop that bench.py's kernel_us times (the first run of at least K launches of",
             "that kernel with no other kernel between them), beside kernel_us itself (HIP events at the ends of",
             "the loop on the launch stream: the kernel plus one launch gap).  roofline.frac is combine's",
             "algorithmic bytes per launch over kernel_us[combine]; recomputed over the profiler's",
             "back-to-back mean it is the 'frac_from_profile' column.  Under the tracer every launch costs",
             "several microseconds more, which inflates the back-to-back figure of a kernel as short as the",
             "layout; the prefill dispatch and combine are long enough not to notice.", "", "commands:",
             PROFILE_COMMANDS,
             "%-52s %6s %11s %6s %11s %10s %7s %9s" % ("kernel", "calls", "avg_all_us", "b2b_n", "avg_b2b_us",
                                                     "bench_us", "ratio", "frac_prof")]
    alg = dict(zip(("layout", "dispatch", "combine"), alg_bytes(4096, 7168, 256, 8, True)))
    alg["layout_dispatch"] = alg["layout"] + alg["dispatch"]
    for step, kern in PROFILED_KERNELS.items():
        r = stats.get(kern)
        if r is None:
            continue
        prof_us = float(r["AverageNs"]) / 1e3
        run = b2b_run(kern, rec["steps"])
        b2b_us = sum(run) / len(run) / 1e3 if run else float("nan")
        bench_us = rec["kernel_us"][step]
        lines.append("%-52s %6s %11.2f %6d %11.2f %10.2f %7.3f %9.4f"
                     % (kern[:52], r["Calls"], prof_us, len(run), b2b_us, bench_us, bench_us / b2b_us,
                        alg[step] / b2b_us / 1e3 / PEAK_HBM_GBS))
    lines += ["", "bench line of that run: value %s %s, us_per_step %s, roofline %s"
              % (rec["value"], rec["unit"], rec["us_per_step"], json.dumps(rec["roofline"]))]
    with open(os.path.join(PROFILES, BENCH_RUN_FILE), "w") as f:
        f.write("\n".join(lines) + "\n")
    return True


WORKLOAD_NOTES = {
    "prefill": "4096 tokens x hidden 7168, 256 experts (8 groups, top-4 groups), top-8, FP8 E4M3 dispatch "
               "(1 scale / 128 ch) + BF16 combine",
    "skew": "4096 tokens x hidden 7168, 256 experts, top-8 from Zipf(1.2) expert popularity, Dirichlet(1) "
            "weights, FP8 E4M3 dispatch + BF16 combine",
    "hbm": "32768 tokens x hidden 7168, 256 experts (8 groups, top-4 groups), top-8, BF16 dispatch (3.76 GB "
           "receive buffer) + BF16 combine of that buffer (identity expert)",
    "decode": "128 tokens x hidden 7168, 256 experts (8 groups, top-4 groups), top-8, FP8 E4M3 dispatch + "
              "BF16 combine",
    "tiny": "64 tokens x hidden 256, 16 experts, top-2, FP8 E4M3 dispatch + BF16 combine",
}


def workload_record(ep, torch, name, steps, warmup, flushed_reps):
    """A configuration's step (ep_layout_dispatch, then ep_combine) timed as
    the headline is: single steps after an Infinity Cache flush (median,
    p10, p90), K back-to-back steps warm, and each call's mean over K
    back-to-back launches.  Rates are algorithmic bytes per second; a call's
    `frac` is its rate over the 8 TB/s peak."""
    s = Setup(ep, torch, name, 0)
    wl = s.wl
    lay_b, dis_b, com_b = s.bytes
    total = lay_b + dis_b + com_b
    warm_us = time_loop(torch, s.step_fused, steps, warmup)
    fl = step_times(torch, s.step_fused, flushed_reps, FLUSH_BYTES)
    plan = s.bare()
    calls = {"layout_dispatch": (plan.layout_dispatch, lay_b + dis_b), "combine": (plan.combine, com_b)}
    if wl.T * wl.K > 65536:  # the one call is then the layout kernels followed by the dispatch kernels
        calls["layout"] = (plan.layout, lay_b)
        calls["dispatch"] = (plan.dispatch, dis_b)
    kus = {k: time_loop(torch, fn, steps, 1) for k, (fn, _) in calls.items()}
    med = pct(fl, 0.5)
    rec = {"config": {"workload": WORKLOAD_NOTES[name] + ", seed 0", "tokens": wl.T, "hidden": wl.H,
                      "experts": wl.E, "top_k": wl.K, "dispatch": "fp8" if wl.fp8 else "bf16"},
           "alg_bytes_per_step": total,
           "us_per_step_flushed": dist(fl),
           "GBs_flushed_median": round(total / med / 1e3, 1),
           "us_per_step_warm": round(warm_us, 2),
           "GBs_warm": round(total / warm_us / 1e3, 1),
           "kernel_us": {k: round(v, 2) for k, v in kus.items()},
           "kernel_alg_bytes": {k: b for k, (_, b) in calls.items()},
           "kernel_GBs": {k: round(calls[k][1] / v / 1e3, 1) for k, v in kus.items()},
           "kernel_frac": {k: round(calls[k][1] / v / 1e3 / PEAK_HBM_GBS, 4) for k, v in kus.items()}}
    del s, plan
    torch.cuda.empty_cache()
    return rec


def other_workload(ep, torch, args):
    """One JSON line for a non-headline configuration (same timing method)."""
    rec = workload_record(ep, torch, args.workload, args.steps, args.warmup, args.steps)
    rec = dict({"metric": "step µs and algorithmic GB/s (ep_layout_dispatch + ep_combine)",
                "workload": args.workload}, **rec)
    print(json.dumps(rec), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-replays", type=int, default=500)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "skew", "hbm", "decode", "tiny"],
                    help="time another configuration (one short JSON line; the default is the headline)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", nargs="?", const="prefill", default=None,
                    choices=["tiny", "decode", "prefill", "skew", "hbm"])
    ap.add_argument("--summarize-profile", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path is one GPU's share with every expert resident in its "
              "HBM, and this library has no multi-GPU transport (requested --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    import combine_ep_dispatch_amd as ep

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.profile_pass:
        profile_pass(ep, torch, args.profile_pass)
        return 0

    if args.workload != "prefill":
        return other_workload(ep, torch, args)

    s = Setup(ep, torch, "prefill", 0)
    lay_b, dis_b, com_b = s.bytes
    total_b = lay_b + dis_b + com_b
    # the headline: K single steps, each after an Infinity Cache flush (the
    # flush outside the step's events), median; then K back-to-back steps
    # warm, each call's back-to-back launches, and the three-call form
    fl = step_times(torch, s.step_fused, args.steps, FLUSH_BYTES, warmup=args.warmup)
    us_step = pct(fl, 0.5)
    us_warm, per_kernel, wall = time_steps(torch, s, args.steps, args.warmup, fused=True)
    us_three = time_loop(torch, s.step, args.steps, args.warmup)
    warm_single = step_times(torch, s.step_fused, args.steps)
    # each call of the step timed alone, in both modes
    call_dist = {name: {"flushed": dist(step_times(torch, fn, args.steps, FLUSH_BYTES)),
                        "warm": dist(step_times(torch, fn, args.steps))}
                 for name, fn in (("layout_dispatch", s.layout_dispatch), ("combine", s.combine))}
    graph_us = time_graph(torch, s.step_fused, 50)
    s.backward_buffers(torch)
    db_b, cb_b = backward_bytes(s.wl.T, s.wl.H, s.wl.K)
    db_us = time_loop(torch, s.dispatch_backward, 30, 3)
    cb_us = time_loop(torch, s.combine_backward, 30, 3)
    wl_prefill = s.wl
    del s
    torch.cuda.empty_cache()
    workloads = {"skew": workload_record(ep, torch, "skew", args.steps, args.warmup, args.steps),
                 "hbm": workload_record(ep, torch, "hbm", 10, 2, 10)}

    # decode: three calls (layout, dispatch, combine), then the fused form
    # (layout + dispatch in one launch, then combine), each eager through
    # the checked binding, eager through StepPlan (buffers checked once) and
    # as a replayed HIP graph; packed and low-latency padded layouts
    decode = {}
    for cap in (0, 128):
        d = Setup(ep, torch, "decode", 0, capacity=cap)
        d_us, d_per, _ = time_steps(torch, d, 200, 10)
        rec_d = {"stream": round(d_us, 2), "graph": round(time_graph(torch, d.step, args.decode_replays), 2),
                 "kernel_us": {k: round(v, 2) for k, v in d_per.items()}}
        plan = d.bare()
        rec_d["fused"] = {"stream": round(time_loop(torch, d.step_fused, 200, 10), 2),
                          "stream_step_plan": round(time_loop(torch, plan.step, 200, 10), 2),
                          "graph": round(time_graph(torch, d.step_fused, args.decode_replays), 2),
                          # one graph launch costs more host time than this step's GPU time;
                          # ten steps in one graph amortise it
                          "graph_10_steps": round(time_graph(torch, d.step_fused, args.decode_replays // 10, 10), 2),
                          "graph_40_steps": round(time_graph(torch, d.step_fused, max(1, args.decode_replays // 40),
                                                             40), 2),
                          "host_us_per_step_step_plan": round(host_submit_us(torch, plan.step, 2000), 2),
                          "kernel_us": {"layout_dispatch": round(time_loop(torch, plan.layout_dispatch, 200, 10), 2)}}
        decode[cap] = rec_d
        del d, plan

    comb_us = per_kernel["combine"]
    achieved = com_b / (comb_us * 1e-6) / 1e9
    traffic = read_traffic()
    rec = {
        "metric": METRIC,
        "value": round(total_b / us_step / 1e3, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3/bf16 storage, f32 arithmetic",
        "data": "synthetic",
        "config": {"workload": "prefill: " + WORKLOAD_NOTES["prefill"] + ", seed 0",
                   "tokens": wl_prefill.T, "hidden": wl_prefill.H, "experts": wl_prefill.E, "top_k": wl_prefill.K},
        "value_method": "algorithmic bytes of one step (830.2 MB) / median of K single steps, each timed with HIP "
                        "events on the launch stream after a 512 MB device read that evicts the Infinity Cache",
        "us_per_step": round(us_step, 2),
        "step": "ep_layout_dispatch (layout + FP8 dispatch, one launch) + ep_combine",
        "us_per_step_warm": round(us_warm, 2),
        "GBs_warm": round(total_b / us_warm / 1e3, 1),
        "us_per_step_graph": round(graph_us, 2),
        "us_per_step_three_calls": round(us_three, 2),
        "step_distribution_us": {"flushed": dist(fl), "warm": dist(warm_single),
                                 "note": "K steps each timed alone (events at the step's two ends only); "
                                         "flushed: a 512 MB device read before every step"},
        "call_distribution_us": dict(call_dist, note="each call alone between two events, K times: p10 / "
                                                      "median / p90; flushed as for the step"),
        "kernel_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "kernel_us_method": "mean of K back-to-back launches of each kernel, HIP events on the launch stream "
                            "(kernel plus one launch gap); layout and dispatch are the three-call form's kernels",
        "kernel_alg_bytes": {"layout_dispatch": lay_b + dis_b, "combine": com_b, "layout": lay_b,
                             "dispatch": dis_b},
        "workloads": workloads,
        "decode_us_per_step": decode[0]["fused"]["stream_step_plan"],
        "decode_step": "128 tokens x 7168, 256 experts, top-8, FP8: ep_layout_dispatch + ep_combine through "
                       "StepPlan, eager, mean of 200 back-to-back steps (HIP events on the launch stream); eager "
                       "decode is host-bound (decode_128tok_us.fused.host_us_per_step_step_plan: host time to "
                       "submit a step, about two HIP kernel launches); graph_40_steps is the GPU time per step "
                       "with the host out of the way",
        "decode_128tok_us": dict(decode[0], low_latency_padded_128=decode[128]),
        "backward_us": {"dispatch_backward": round(db_us, 2), "combine_backward": round(cb_us, 2),
                        "dispatch_backward_GBs": round(db_b / db_us / 1e3, 1),
                        "combine_backward_GBs": round(cb_b / cb_us / 1e3, 1)},
        "roofline": {"bound": "hbm", "kernel": "combine", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic["combine"] if traffic else None,
                     "achieved_method": "combine's algorithmic bytes per launch (528.7 MB, 4096 tokens) / "
                                        "kernel_us[combine]",
                     "traffic_source": "committed rocprofv3 FETCH_SIZE + WRITE_SIZE summary (%s), used only "
                                       "while every kernel source hashes as it did when the counters were "
                                       "taken" % os.path.relpath(TRAFFIC_FILE, ROOT)},
    }
    if traffic is not None:
        # each kernel's mean launch duration over the bytes the HBM counters saw
        rec["roofline"]["traffic_GBs"] = round(traffic["combine"] / (comb_us * 1e-6) / 1e9, 1)
        rec["counter_bytes_per_launch"] = {k: int(v) for k, v in traffic.items()}
        rec["counter_GBs"] = {k: round(traffic[k] / (per_kernel[k] * 1e-6) / 1e9, 1) for k in traffic}
        rec["counter_GBs_step"] = round(sum(traffic[k] for k in STEP_KERNELS) / (us_step * 1e-6) / 1e9, 1)
    rec["context_pages"] = {
        "note": "DeepEP on H800, multi-GPU all-to-all over interconnects; context, not a target",
        "normal_kernels_nvlink_GBs": "153-158", "normal_kernels_rdma_GBs": "43-47",
        "low_latency_us": 163, "low_latency_rdma_GBs": "39-46"}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl_prefill, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
