"""The FP8 quantiser divides a group's 128 channels by their shared scale
with one correctly rounded reciprocal and an FMA correction per channel
(csrc/ep_device.h, div_by_recip), in place of 128 full divisions.  Its
results must be those of IEEE division, which the oracle uses.  This test
compiles a C check of that arithmetic with gcc and runs it on the CPU:
exhaustive over every BF16 significand (two binades) against every binary32
divisor significand, sampled over exponents, plus the tiny-channel and
signed-zero cases (tests/c_abi/shared_divisor_check.c says which).  The
GPU parity tests then hold the kernels themselves to the oracle."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div") / "shared_divisor_check")
    src = os.path.join(ROOT, "tests", "c_abi", "shared_divisor_check.c")
    # hardware FMA where the CPU has it (glibc's fmaf is correctly rounded
    # either way, only slower); no contraction of a*y into an FMA
    flags = ["-O2", "-ffp-contract=off", "-Wall", "-Werror"] + (["-mfma"] if _has_fma() else [])
    r = subprocess.run(["gcc", *flags, src, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_shared_divisor_matches_ieee_division(checker):
    r = subprocess.run([checker], capture_output=True, text=True, timeout=600)
    f = r.stdout.split()
    got = dict(zip(f[0::2], (int(v) for v in f[1::2])))
    assert got["pairs"] == 256 * (1 << 23)
    assert got["q0_wrong"] > 0, "the uncorrected quotient should differ somewhere: the check would be vacuous"
    assert got["q1_wrong"] == 0
    assert got["sampled"] == 20000000 and got["sample_wrong"] == 0
    assert got["tiny"] > 100000 and got["tiny_wrong"] == 0
    assert got["zero_wrong"] == 0
    assert r.returncode == 0
