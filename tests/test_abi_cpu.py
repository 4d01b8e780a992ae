"""The C-ABI library loads and exports what include/ep.h declares (CPU only).

Only host-side paths run here: argument checks that return before any
launch, the workspace-size query and the status strings.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import combine_ep_dispatch_amd as ep

    return ep


def test_header_declares_the_three_calls():
    names = declared_functions()
    for f in ("ep_dispatch_layout", "ep_dispatch", "ep_combine"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(lib._lib.EXPORTS)


def test_status_strings(lib):
    s = lib.LIB.ep_status_string
    assert s(0) == b"EP_OK" and s(1) == b"EP_ERR_INVALID_ARG"
    assert s(2) == b"EP_ERR_UNSUPPORTED" and s(3) == b"EP_ERR_HIP" and s(99) == b"EP_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    f = lib.ep_layout_workspace_bytes
    assert f(64, 2, 16) == 0          # single workgroup
    assert f(128, 8, 256) == 0
    assert f(4096, 8, 256) == 0       # single-launch paths up to 65536 entries
    assert f(8192, 8, 256) == 0
    assert f(8193, 8, 256) == 17 * 257 * 4  # then 4096-entry chunks
    assert f(65537, 1, 1024) == 17 * 1025 * 4
    assert f(32768, 8, 256) == 64 * 257 * 4
    assert f(-1, 8, 256) == 0 and f(10, 0, 4) == 0 and f(10, 2, 2000) == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_layout_rejects_bad_arguments(lib):
    L = lib.LIB.ep_dispatch_layout
    ok = dict(idx=FAKE, T=4, K=2, E=8, c=FAKE, o=FAKE, s=FAKE, r=FAKE, ws=None, wsb=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L(a["idx"], a["T"], a["K"], a["E"], a["c"], a["o"], a["s"], a["r"], a["ws"], a["wsb"], None)

    assert call(K=0) == lib.EP_ERR_INVALID_ARG
    assert call(T=-1) == lib.EP_ERR_INVALID_ARG
    assert call(E=0) == lib.EP_ERR_INVALID_ARG
    assert call(E=1025) == lib.EP_ERR_UNSUPPORTED
    assert call(K=33) == lib.EP_ERR_UNSUPPORTED
    assert call(c=None) == lib.EP_ERR_INVALID_ARG
    assert call(idx=None) == lib.EP_ERR_INVALID_ARG
    assert call(s=FAKE + 2) == lib.EP_ERR_INVALID_ARG  # misaligned int32
    assert call(T=1 << 20, K=8) == lib.EP_ERR_UNSUPPORTED  # beyond 2**22 entries
    # multi-block shapes need a workspace
    assert call(T=8200, K=8, E=256) == lib.EP_ERR_INVALID_ARG
    assert call(T=8200, K=8, E=256, ws=FAKE, wsb=100) == lib.EP_ERR_INVALID_ARG
    assert call(T=8200, K=8, E=256, ws=FAKE + 4, wsb=1 << 20) == lib.EP_ERR_INVALID_ARG  # misaligned


def test_dispatch_and_combine_reject_bad_arguments(lib):
    D = lib.LIB.ep_dispatch
    C = lib.LIB.ep_combine
    fp8, bf16 = lib.EP_RECV_FP8_E4M3_G128, lib.EP_RECV_BF16
    assert D(FAKE, 4, 200, 2, FAKE, None, fp8, FAKE, FAKE, None, None) == lib.EP_ERR_INVALID_ARG  # H%128
    assert D(FAKE, 4, 130, 2, FAKE, None, bf16, FAKE, None, None, None) == lib.EP_ERR_INVALID_ARG  # H%8
    assert D(FAKE, 4, 256, 2, FAKE, None, 7, FAKE, FAKE, None, None) == lib.EP_ERR_INVALID_ARG
    assert D(FAKE, 4, 256, 2, FAKE, None, fp8, FAKE, None, None, None) == lib.EP_ERR_INVALID_ARG  # no scale
    assert D(FAKE + 8, 4, 256, 2, FAKE, None, fp8, FAKE, FAKE, None, None) == lib.EP_ERR_INVALID_ARG
    assert D(FAKE, 4, 256, 2, FAKE, None, fp8, FAKE, FAKE, FAKE, None) == lib.EP_ERR_INVALID_ARG  # w needed
    assert D(None, 0, 256, 2, None, None, fp8, None, None, None, None) == lib.EP_OK  # T == 0: no-op
    assert C(FAKE, FAKE, FAKE, 4, 12, 2, FAKE, None) == lib.EP_ERR_INVALID_ARG  # H%8
    assert C(FAKE, FAKE, None, 4, 16, 2, FAKE, None) == lib.EP_ERR_INVALID_ARG
    assert C(FAKE, FAKE, FAKE, 4, 16, 0, FAKE, None) == lib.EP_ERR_INVALID_ARG
    assert C(None, None, None, 0, 16, 2, None, None) == lib.EP_OK
    assert lib.LIB.ep_cast_fp8_e4m3(FAKE, FAKE + 1, 8, None) == lib.EP_ERR_INVALID_ARG
    assert lib.LIB.ep_cast_fp8_e4m3(None, None, 0, None) == lib.EP_OK


def test_size_limits_keep_launches_in_range(lib):
    """T*H reaches 2**34 (2**21 tokens of hidden 8192, top-1): every call that
    launches T*H/8 or T*H/16 work items refuses it, as the FP8 cast refuses
    n = 2**33, so no launch reaches 2**31 work items."""
    L, U = lib.LIB, lib.EP_ERR_UNSUPPORTED
    T, H, fp8 = 1 << 21, 8192, lib.EP_RECV_FP8_E4M3_G128
    assert L.ep_dispatch(FAKE, T, H, 1, FAKE, None, fp8, FAKE, FAKE, None, None) == U
    assert L.ep_dispatch(FAKE, T, H, 1, FAKE, None, lib.EP_RECV_BF16, FAKE, None, None, None) == U
    assert L.ep_combine(FAKE, FAKE, FAKE, T, H, 1, FAKE, None) == U
    assert L.ep_dispatch_backward(FAKE, FAKE, T, H, 1, FAKE, None) == U
    assert L.ep_combine_backward(FAKE, FAKE, FAKE, FAKE, T, H, 1, FAKE, None, None) == U
    ws = lib.ep_layout_workspace_bytes(T, 1, 8)
    assert L.ep_layout_dispatch(FAKE, FAKE, None, T, H, 1, 8, 0, fp8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                FAKE, ws, None) == U
    assert L.ep_cast_fp8_e4m3(FAKE, FAKE, 1 << 33, None) == U


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "combine_ep_dispatch_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", text), f


def test_padded_layout_rejects_bad_arguments(lib):
    P = lib.LIB.ep_dispatch_layout_padded

    def call(T=4, K=2, E=8, cap=16, cnt=FAKE, s=FAKE, r=FAKE, idx=FAKE):
        return P(idx, T, K, E, cap, cnt, s, r, None, 0, None)

    assert call(cap=0) == lib.EP_ERR_INVALID_ARG
    assert call(E=1024, cap=1 << 21) == lib.EP_ERR_INVALID_ARG  # E*cap >= 2**31
    assert call(cnt=None) == lib.EP_ERR_INVALID_ARG
    assert call(r=None) == lib.EP_ERR_INVALID_ARG
    assert call(s=None) == lib.EP_ERR_INVALID_ARG
    assert call(E=2000) == lib.EP_ERR_UNSUPPORTED
    assert call(T=8200, K=8, E=256) == lib.EP_ERR_INVALID_ARG  # needs a workspace


def test_step_plan_rejects_host_tensors():
    """StepPlan validates its buffers before any C call (no GPU needed)."""
    import torch
    ep = pytest.importorskip("combine_ep_dispatch_amd")
    idx = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.ones((4, 2), dtype=torch.float32)
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU device"):
        ep.StepPlan(idx, w, x, 8)


def test_layout_dispatch_rejects_bad_arguments(lib):
    """ep_layout_dispatch checks the union of the layout and dispatch
    arguments; every call below fails validation before any launch."""
    F = lib.LIB.ep_layout_dispatch
    fp8, bf16 = lib.EP_RECV_FP8_E4M3_G128, lib.EP_RECV_BF16
    ok = dict(idx=FAKE, x=FAKE, w=None, T=4, H=256, K=2, E=8, cap=0, fmt=fp8, c=FAKE, o=FAKE, s=FAKE, r=FAKE,
              rx=FAKE, rs=FAKE, rw=None, ws=None, wsb=0)

    def call(**kw):
        a = dict(ok, **kw)
        return F(a["idx"], a["x"], a["w"], a["T"], a["H"], a["K"], a["E"], a["cap"], a["fmt"], a["c"], a["o"],
                 a["s"], a["r"], a["rx"], a["rs"], a["rw"], a["ws"], a["wsb"], None)

    bad = lib.EP_ERR_INVALID_ARG
    assert call(K=0) == bad and call(T=-1) == bad and call(E=0) == bad and call(cap=-1) == bad
    assert call(E=1025) == lib.EP_ERR_UNSUPPORTED and call(K=33) == lib.EP_ERR_UNSUPPORTED
    assert call(o=None) == bad                       # packed layout needs offsets
    assert call(cap=4, r=None) == bad                # padded layout needs src
    assert call(cap=1 << 21, E=1024) == bad          # E*cap >= 2**31
    assert call(c=None) == bad and call(idx=None) == bad and call(s=FAKE + 2) == bad
    assert call(H=200) == bad                        # FP8 needs H % 128 == 0
    assert call(H=130, fmt=bf16) == bad              # H % 8
    assert call(fmt=7) == bad
    assert call(rs=None) == bad                      # FP8 needs the scales
    assert call(x=FAKE + 8) == bad                   # 16-byte alignment
    assert call(rw=FAKE) == bad                      # recv_weight needs topk_weights
    assert call(T=8200, K=8, E=256) == bad           # past 65536 entries the workspace is required
    assert call(T=1 << 20, K=8) == lib.EP_ERR_UNSUPPORTED


def test_header_is_strict_c():
    """include/ep.h is a C header: it compiles as strict C99 on its own."""
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c",
                        HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_driver_compiles_and_links(lib, tmp_path):
    """The plain-C test driver builds against include/ep.h and links every
    call it makes against libep.so."""
    import importlib.util
    import subprocess
    spec = importlib.util.spec_from_file_location("_c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    r = subprocess.run(mod.command(str(tmp_path / "ep_step")), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_int64_id_calls_reject_bad_arguments(lib):
    """The int64-id entry points check what the int32 ones do, with the ids
    aligned to 8 bytes."""
    L = lib.LIB.ep_dispatch_layout_i64
    P = lib.LIB.ep_dispatch_layout_padded_i64
    F = lib.LIB.ep_layout_dispatch_i64
    bad = lib.EP_ERR_INVALID_ARG
    assert L(FAKE + 4, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == bad  # 4-byte aligned ids
    assert L(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == bad
    assert L(FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, FAKE, None, 0, None) == lib.EP_ERR_UNSUPPORTED
    assert P(FAKE + 4, 4, 2, 8, 16, FAKE, FAKE, FAKE, None, 0, None) == bad
    assert P(FAKE, 4, 2, 8, 0, FAKE, FAKE, FAKE, None, 0, None) == bad
    fp8 = lib.EP_RECV_FP8_E4M3_G128
    assert F(FAKE + 4, FAKE, None, 4, 256, 2, 8, 0, fp8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
             None) == bad
    assert F(FAKE, FAKE, None, 4, 200, 2, 8, 0, fp8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
             None) == bad  # H % 128


def test_noalloc_layout_dispatch_rejects_bad_arguments_and_oversize(lib):
    """ep_layout_dispatch_noalloc checks what ep_layout_dispatch checks
    (without a workspace) and refuses, before touching the device, shapes
    whose layout histograms do not fit its fixed scratch."""
    F = lib.LIB.ep_layout_dispatch_noalloc
    fp8 = lib.EP_RECV_FP8_E4M3_G128
    ok = dict(idx=FAKE, x=FAKE, w=None, T=4, H=256, K=2, E=8, cap=0, fmt=fp8, c=FAKE, o=FAKE, s=FAKE, r=FAKE,
              rx=FAKE, rs=FAKE, rw=None)

    def call(**kw):
        a = dict(ok, **kw)
        return F(a["idx"], a["x"], a["w"], a["T"], a["H"], a["K"], a["E"], a["cap"], a["fmt"], a["c"], a["o"],
                 a["s"], a["r"], a["rx"], a["rs"], a["rw"], None)

    bad, uns = lib.EP_ERR_INVALID_ARG, lib.EP_ERR_UNSUPPORTED
    assert call(K=0) == bad and call(T=-1) == bad and call(E=0) == bad
    assert call(o=None) == bad and call(idx=None) == bad and call(rs=None) == bad
    assert call(H=200) == bad and call(x=FAKE + 8) == bad
    assert call(E=1025) == uns and call(K=33) == uns and call(T=1 << 20, K=8) == uns
    # the scratch holds (E+1) int32 per 4096-entry chunk, 1 MiB in all
    assert lib.EP_NOALLOC_SCRATCH_BYTES == 1 << 20
    assert lib.ep_layout_workspace_bytes(1044480, 1, 1024) <= lib.EP_NOALLOC_SCRATCH_BYTES
    assert lib.ep_layout_workspace_bytes(1044481, 1, 1024) > lib.EP_NOALLOC_SCRATCH_BYTES
    assert call(T=1044481, K=1, E=1024, H=128) == uns
    assert call(T=(1 << 22) // 8, K=8, E=256, H=128) == uns
    assert call(T=1 << 19, K=8, E=8, cap=0, H=128, fmt=fp8, idx=None) == bad  # still checked first


def test_step_plan_init_checks_and_guards(lib):
    """ep_step_plan_init checks what ep_layout_dispatch and ep_combine check;
    a plan that was never initialised, or whose init failed, launches
    nothing.  (Only host paths run: no plan here reaches a launch.)"""
    L = lib.LIB
    plan = (ctypes.c_uint64 * lib._lib.STEP_PLAN_WORDS)()
    pp = ctypes.c_void_p(ctypes.addressof(plan))
    fp8 = lib.EP_RECV_FP8_E4M3_G128
    ok = dict(idx=FAKE, ib=4, x=FAKE, w=FAKE, T=4, H=256, K=2, E=8, cap=0, fmt=fp8, c=FAKE, o=FAKE, s=FAKE, r=FAKE,
              rx=FAKE, rs=FAKE, rw=None, ws=None, wsb=0, y=FAKE, out=FAKE)

    def init(**kw):
        a = dict(ok, **kw)
        return L.ep_step_plan_init(pp, a["idx"], a["ib"], a["x"], a["w"], a["T"], a["H"], a["K"], a["E"], a["cap"],
                                   a["fmt"], a["c"], a["o"], a["s"], a["r"], a["rx"], a["rs"], a["rw"], a["ws"],
                                   a["wsb"], a["y"], a["out"], None)

    bad, uns = lib.EP_ERR_INVALID_ARG, lib.EP_ERR_UNSUPPORTED
    # never initialised: zero storage launches nothing
    assert L.ep_step_plan_layout_dispatch(pp) == bad and L.ep_step_plan_combine(pp) == bad
    assert L.ep_step_plan_layout_dispatch(None) == bad and L.ep_step_plan_combine(None) == bad
    assert L.ep_step_plan_init(None, FAKE, 4, FAKE, FAKE, 4, 256, 2, 8, 0, fp8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None, 0, FAKE, FAKE, None) == bad
    assert init() == lib.EP_OK
    assert init(ib=2) == bad and init(ib=8, idx=FAKE + 4) == bad
    # a failed init leaves the plan unusable, even after a good one
    assert L.ep_step_plan_layout_dispatch(pp) == bad and L.ep_step_plan_combine(pp) == bad
    # the layout + dispatch checks
    assert init(K=0) == bad and init(E=1025) == uns and init(o=None) == bad and init(rs=None) == bad
    assert init(H=200) == bad and init(x=FAKE + 8) == bad and init(T=8200, K=8, E=256) == bad
    # the combine checks: y and out both or neither; weights; alignment
    assert init(y=None) == bad and init(out=None) == bad and init(out=FAKE + 2) == bad
    assert init(w=None) == bad
    assert init(y=None, out=None) == lib.EP_OK      # layout + dispatch only
    assert L.ep_step_plan_combine(pp) == bad        # ... so no combine
    assert init(T=0, y=None, out=None, w=None) == lib.EP_OK
    assert L.ep_step_plan_combine(pp) == lib.EP_OK  # an empty batch: nothing to reduce
