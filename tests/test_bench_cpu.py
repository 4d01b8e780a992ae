"""bench.py's host-side logic on the CPU: the algorithmic byte counts, the
refusal of more than one GPU, and the rocprofv3 summariser (counter
calibration, per-launch bytes, the source-hash guard) on a small synthetic
profiler output."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_match_the_tabulated_totals():
    """Totals per configuration as tabulated from the byte formulas when the
    workloads were specified (MB = 1e6 bytes, three significant decimals)."""
    def mb(v):
        return round(v / 1e6, 2)

    lay, dis, com = bench.alg_bytes(4096, 7168, 256, 8, True)
    assert (round(lay / 1e6, 3), mb(dis), mb(com), round((lay + dis + com) / 1e6, 1)) == (0.395, 301.07, 528.74,
                                                                                            830.2)
    lay, dis, com = bench.alg_bytes(128, 7168, 256, 8, True)
    assert (round(lay / 1e6, 3), mb(dis), mb(com), mb(lay + dis + com)) == (0.014, 9.41, 16.52, 25.95)
    lay, dis, com = bench.alg_bytes(32768, 7168, 256, 8, False)
    assert (mb(lay), round(dis / 1e6, 1), round(com / 1e6, 1), round((lay + dis + com) / 1e6)) == (3.15, 4228.9,
                                                                                                   4230.0, 8462)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summarizer_scales_counters_and_guards_by_source_hash(tmp_path, monkeypatch):
    out, prof = tmp_path / "out", tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof / "traffic.txt"))
    names = {k: "void ep::(anonymous namespace)::%s(int const*)" % v for k, v in bench.PROFILED_KERNELS.items()}
    copy = "__amd_rocclr_copyBuffer"
    _write_csv(str(out / "prof_trace" / "t_kernel_stats.csv"),
               [{"Name": n, "Calls": 5, "AverageNs": 1000.0 * (i + 1), "MinNs": 900.0, "MaxNs": 1100.0}
                for i, n in enumerate(names.values())])
    # calibration: the 1 GiB copy reads FETCH_SIZE 512 MiB (scale 2) and WRITE_SIZE 1 GiB (scale 1)
    fetch = {copy: 524288.0, names["layout"]: 100.0, names["dispatch"]: 29000.0, names["combine"]: 230000.0,
             names["layout_dispatch"]: 29500.0}
    write = {copy: 1048576.0, names["layout"]: 50.0, names["dispatch"]: 236000.0, names["combine"]: 57000.0,
             names["layout_dispatch"]: 236500.0}
    for sub, counter, vals in (("prof_fetch", "FETCH_SIZE", fetch), ("prof_write", "WRITE_SIZE", write)):
        rows = []
        for n, v in vals.items():
            rows += [{"Kernel_Name": n, "Counter_Name": counter, "Counter_Value": v}] * 2
        _write_csv(str(out / sub / "c_counter_collection.csv"), rows)
    bench.summarize_profile(str(out))
    text = open(prof / "traffic.txt").read()
    assert "fetch_scale: 2.0000" in text and "write_scale: 1.0000" in text
    got = bench.read_traffic()
    assert set(got) == {"layout_dispatch", "combine", "layout", "dispatch"}
    for step in got:
        assert got[step] == fetch[names[step]] * 1024 * 2 + write[names[step]] * 1024
    # the one-launch kernel is held against the layout's and the dispatch's bytes together
    lay, dis, _ = bench.alg_bytes(4096, 7168, 256, 8, True)
    assert ("algorithmic %12d B" % (lay + dis)) in text
    assert (prof / "prefill_4096x7168_top8_kernel_trace.txt").exists()
    # a source change invalidates the counter bytes
    stale = text.replace("source_sha256: ", "source_sha256: 0")
    with open(prof / "traffic.txt", "w") as f:
        f.write(stale)
    assert bench.read_traffic() is None


def test_bench_run_summary_pairs_profiler_and_bench_line(tmp_path, monkeypatch):
    out, prof = tmp_path / "out", tmp_path / "profiles"
    os.makedirs(prof)
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    stats = [{"Name": "void ep::(anonymous namespace)::%s(int)" % k, "Calls": 100, "AverageNs": ns, "MinNs": ns,
              "MaxNs": ns} for k, ns in zip(bench.PROFILED_KERNELS.values(), (54000.0, 90000.0, 9000.0, 50000.0))]
    _write_csv(str(out / "prof_bench" / "b_kernel_stats.csv"), stats)
    # a trace: two steps (layout_dispatch, combine at 95 us), then 3
    # back-to-back layout launches at 9 us, then 4 back-to-back combines at 90 us
    names = {k: "void ep::(anonymous namespace)::%s(int)" % v for k, v in bench.PROFILED_KERNELS.items()}
    seq = ([("layout_dispatch", 54000), ("combine", 95000)] * 2 + [("layout", 9000)] * 3 + [("combine", 90000)] * 4
           + [("dispatch", 50000)] + [("combine", 99000)] * 6)  # a later, longer run of another workload
    trace, t = [], 1000
    for k, ns in seq:
        trace.append({"Kernel_Name": names[k], "Start_Timestamp": t, "End_Timestamp": t + ns})
        t += ns + 500
    _write_csv(str(out / "prof_bench" / "b_kernel_trace.csv"), trace)
    line = {"value": 1.0, "unit": "GB/s", "us_per_step": 150.0, "roofline": {"frac": 0.7}, "steps": 3,
            "kernel_us": {"layout_dispatch": 53.0, "combine": 88.2, "layout": 9.9, "dispatch": 50.5}}
    with open(out / "bench_under_rocprof.json", "w") as f:
        f.write("some profiler noise\n" + json.dumps(line) + "\n")

    def rows(sub, pattern):
        import glob
        res = []
        for p in glob.glob(os.path.join(str(out), sub, "**", pattern), recursive=True):
            res += list(csv.DictReader(open(p)))
        return res

    assert bench.summarize_bench_run(str(out), rows, lambda n: n.replace("void ep::(anonymous namespace)::", "")
                                     .split("(")[0])
    text = open(prof / bench.BENCH_RUN_FILE).read()
    row = next(ln for ln in text.splitlines() if ln.startswith(bench.STEP_KERNELS["combine"]))
    assert "     4 " in row and " 90.00 " in row and " 0.980 " in row  # 4 back-to-back launches; 88.2 / 90.0
    assert " 0.7344" in row  # 528744448 B / 90.0 us / 8000 GB/s = 0.73437
    row = next(ln for ln in text.splitlines() if ln.startswith(bench.REF_KERNELS["layout"]))
    assert " 1.100 " in row  # layout 9.9 / 9.0
