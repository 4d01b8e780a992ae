"""The burst launch plan (csrc/burst_plan.h) on the CPU: compiled with g++
and checked on device sizes of 32, 128 and 256 CUs (partitions of MI355X
report fewer CUs).  Every launch must fit one wave of workgroups (at most
one per CU), hold at most `items` work items per lane, stay within the
160 KB of LDS a workgroup may take, and the slices must cover the batch
exactly once."""

import itertools
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LDS_LIMIT = 160 * 1024


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "burst_plan_check")
    src = os.path.join(ROOT, "tests", "c_abi", "burst_plan_check.cpp")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", src, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    return exe


def plans(exe, shapes):
    args = [str(v) for s in shapes for v in s]
    out = subprocess.run([exe] + args, capture_output=True, text=True, check=True).stdout.split("\n")
    res, cur = [], None
    for line in out:
        f = line.split()
        if not f:
            continue
        if f[0] == "plan":
            cur = {"launches": int(f[1]), "slice": int(f[2]), "tpb_max": int(f[3]), "slices": []}
            res.append(cur)
        else:
            cur["slices"].append(tuple(int(v) for v in f[1:]))
    assert len(res) == len(shapes)
    return res


def test_fanout_and_combine_plans_fit(planner):
    shapes = []
    for cus, H, K, T in itertools.product((32, 128, 256), (64, 1024, 7168, 8192), (1, 8, 32),
                                          (1, 257, 4096, 32768, 131072)):
        if T * K > 1 << 22:
            continue
        shapes.append((T, H // 8, 14, 1024, cus, 8 * K, LDS_LIMIT))  # fan-out: K rows + K weights per token
        shapes.append((T, H // 8, 14, 1024, cus, 0, 0))              # combine: no LDS
    for shape, p in zip(shapes, plans(planner, shapes)):
        T, vpt, items, threads, cus, lds_tok, _ = shape
        assert p["launches"] > 0, shape
        assert sum(s[0] for s in p["slices"]) == T and len(p["slices"]) == p["launches"], shape
        for Ts, tpb, grid, lds in p["slices"]:
            assert grid <= cus and (grid - 1) * tpb < Ts <= grid * tpb, shape
            assert tpb <= p["tpb_max"] and tpb * vpt <= items * threads, shape
            assert lds <= LDS_LIMIT, shape


def test_lds_caps_tokens_per_workgroup(planner):
    """hidden 64, top-32, 131072 tokens on 128 CUs: registers would allow
    1792 tokens per workgroup, but their rows and weights (256 B each) cap
    it at 640, so the batch goes in two slices instead of one launch that
    asks for 256 KB of LDS."""
    (p,) = plans(planner, [(131072, 8, 14, 1024, 128, 256, LDS_LIMIT)])
    assert p["tpb_max"] == 640 and p["launches"] == 2
    assert all(lds <= LDS_LIMIT for _, _, _, lds in p["slices"])


def test_no_plan_without_cus_or_room(planner):
    shapes = [(4096, 896, 14, 1024, 0, 64, LDS_LIMIT),     # CU count unknown
              (4096, 896, 14, 1024, 256, LDS_LIMIT + 1, LDS_LIMIT),  # one token's LDS does not fit
              (4096, 20000, 14, 1024, 256, 0, 0),          # one token's items do not fit
              (0, 896, 14, 1024, 256, 0, 0)]
    assert [p["launches"] for p in plans(planner, shapes)] == [0, 0, 0, 0]
