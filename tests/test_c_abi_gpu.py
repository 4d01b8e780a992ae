"""One step through the C ABI from plain C (tests/c_abi/ep_step: the HIP
runtime and libep.so, no Python), bit-exact against the oracle.

The C program reads seeded inputs from files, runs the layout call and
ep_dispatch (or ep_layout_dispatch), then ep_combine, and writes every
output back; this test compares them with the oracle's.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import make_workload, to_bf16_bits

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "ep_step")


@pytest.mark.parametrize("ids64", [False, True])
@pytest.mark.parametrize("name,T,cap,mode", [("decode", None, 0, 0), ("decode", None, 0, 1), ("decode", None, 128, 0),
                                             ("decode", None, 128, 1), ("tiny", None, 0, 1), ("tiny", None, 3, 1),
                                             ("prefill", 600, 0, 0), ("prefill", 600, 0, 1), ("decode", None, 0, 2),
                                             ("decode", None, 128, 2), ("tiny", None, 3, 2), ("prefill", 600, 0, 2)])
def test_c_driver_matches_oracle(gpu, tmp_path, name, T, cap, mode, ids64):
    """mode 0: the layout call then ep_dispatch; 1: ep_layout_dispatch; 2:
    an ep_step_plan, its two launches run twice.  ids64: int64 expert ids
    through the *_i64 entry points (mode 2: id_bytes 8)."""
    assert os.path.exists(EXE), "C driver not built: run `python tests/c_abi/build.py`"
    wl = make_workload(name, seed=11, T=T)
    T, H, E, K = wl.T, wl.H, wl.E, wl.K
    rows = E * cap if cap else T * K
    rng = np.random.default_rng(11)
    y = to_bf16_bits(rng.standard_normal((rows, H), dtype=np.float32))
    wl.topk_idx.astype(np.int64 if ids64 else np.int32).tofile(tmp_path / "topk_idx.bin")
    wl.x_bits.astype(np.uint16).tofile(tmp_path / "x.bin")
    wl.topk_weights.astype(np.float32).tofile(tmp_path / "w.bin")
    y.astype(np.uint16).tofile(tmp_path / "y.bin")
    print("case c-abi", name, T, cap, mode, ids64, flush=True)
    r = subprocess.run([EXE, str(tmp_path), str(T), str(H), str(K), str(E), str(cap), str(mode), str(int(ids64))],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    def out(fname, dtype, shape):
        return np.fromfile(tmp_path / fname, dtype=dtype).reshape(shape)

    if cap:
        oc, oslot, osrc = oracle.dispatch_layout_padded(wl.topk_idx, E, cap)
        used = (np.arange(cap)[None, :] < oc[:, None]).ravel()
    else:
        oc, oo, oslot, osrc = oracle.dispatch_layout(wl.topk_idx, E)
        assert np.array_equal(out("offsets.bin", np.int32, (E + 1,)), oo)
        used = np.arange(rows) < oo[-1]
    assert np.array_equal(out("counts.bin", np.int32, (E,)), oc)
    assert np.array_equal(out("slot.bin", np.int32, (T, K)), oslot)
    assert np.array_equal(out("src.bin", np.int32, (rows,))[used], osrc[used])
    orecv, oscale, orw = oracle.dispatch_fp8(wl.x_bits, oslot, num_rows=rows, topk_weights=wl.topk_weights)
    assert np.array_equal(out("recv.bin", np.uint8, (rows, H))[used], orecv[used])
    assert np.array_equal(out("scale.bin", np.uint32, (rows, H // 128))[used], oscale[used].view(np.uint32))
    assert np.array_equal(out("rweight.bin", np.float32, (rows,))[used], orw[used])
    assert np.array_equal(out("out.bin", np.uint16, (T, H)), oracle.combine(y, oslot, wl.topk_weights))
