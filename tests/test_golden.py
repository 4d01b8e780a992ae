"""Fixtures under tests/golden/ (CPU only)."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_ocp_e4m3_spec_points():
    """Encode and decode the OCP OFP8 v1.0 E4M3 table points (cited in the file)."""
    for line in open(os.path.join(GOLDEN, "ocp_e4m3_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        value, code = line.split()
        v = np.float32(float(value))
        c = int(code, 16)
        assert int(oracle.f32_to_e4m3_rne_sat(np.array([v]))[0]) == c, line
        d = oracle.e4m3_to_f32(np.array([c], np.uint8))[0]
        assert d == v and np.signbit(d) == np.signbit(v), line


def test_oracle_digests_unchanged():
    """The oracle's outputs on seeded inputs match the committed digests;
    a mismatch means its arithmetic or the generators changed."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(GOLDEN, "oracle_digests.json")) as f:
        want = json.load(f)
    assert mod.compute() == want
