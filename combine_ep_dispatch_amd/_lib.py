"""ctypes loader for libep.so, the C-ABI library declared in include/ep.h.

Loading fails loudly (ImportError) when the library has not been built:
there is no fallback path.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libep.so")

EP_OK = 0
EP_ERR_INVALID_ARG = 1
EP_ERR_UNSUPPORTED = 2
EP_ERR_HIP = 3

EP_RECV_FP8_E4M3_G128 = 0
EP_RECV_BF16 = 1

EP_MAX_EXPERTS = 1024
EP_MAX_TOPK = 32
EP_NOALLOC_SCRATCH_BYTES = 1 << 20

# ep_step_plan: opaque caller-owned storage of 32 uint64
STEP_PLAN_WORDS = 32

EXPORTS = (
    "ep_status_string",
    "ep_layout_workspace_bytes",
    "ep_dispatch_layout",
    "ep_dispatch_layout_i64",
    "ep_dispatch_layout_padded",
    "ep_dispatch_layout_padded_i64",
    "ep_dispatch",
    "ep_layout_dispatch",
    "ep_layout_dispatch_i64",
    "ep_layout_dispatch_noalloc",
    "ep_combine",
    "ep_step_plan_init",
    "ep_step_plan_layout_dispatch",
    "ep_step_plan_combine",
    "ep_dispatch_backward",
    "ep_combine_backward",
    "ep_cast_fp8_e4m3",
)


class EpError(RuntimeError):
    def __init__(self, fn, status, lib):
        self.status = status
        name = lib.ep_status_string(status).decode()
        super().__init__("%s failed: %s (%d)" % (fn, name, status))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libep.so is not built (%s); run `python combine_ep_dispatch_amd/build.py`" % LIB_PATH)
    # torch first, so that the HIP runtime the library links against is the
    # one torch already holds
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.ep_status_string.argtypes = [ctypes.c_int]
    lib.ep_status_string.restype = ctypes.c_char_p
    lib.ep_layout_workspace_bytes.argtypes = [i64, i32, i32]
    lib.ep_layout_workspace_bytes.restype = sz
    for suffix in ("", "_i64"):
        getattr(lib, "ep_dispatch_layout" + suffix).argtypes = [p, i64, i32, i32, p, p, p, p, p, sz, p]
        getattr(lib, "ep_dispatch_layout" + suffix).restype = ctypes.c_int
        getattr(lib, "ep_dispatch_layout_padded" + suffix).argtypes = [p, i64, i32, i32, i32, p, p, p, p, sz, p]
        getattr(lib, "ep_dispatch_layout_padded" + suffix).restype = ctypes.c_int
        getattr(lib, "ep_layout_dispatch" + suffix).argtypes = [p, p, p, i64, i32, i32, i32, i32, i32, p, p, p, p, p,
                                                                p, p, p, sz, p]
        getattr(lib, "ep_layout_dispatch" + suffix).restype = ctypes.c_int
    lib.ep_layout_dispatch_noalloc.argtypes = [p, p, p, i64, i32, i32, i32, i32, i32, p, p, p, p, p, p, p, p]
    lib.ep_layout_dispatch_noalloc.restype = ctypes.c_int
    lib.ep_dispatch.argtypes = [p, i64, i32, i32, p, p, i32, p, p, p, p]
    lib.ep_dispatch.restype = ctypes.c_int
    lib.ep_combine.argtypes = [p, p, p, i64, i32, i32, p, p]
    lib.ep_combine.restype = ctypes.c_int
    lib.ep_step_plan_init.argtypes = [p, p, i32, p, p, i64, i32, i32, i32, i32, i32, p, p, p, p, p, p, p, p, sz, p,
                                      p, p]
    lib.ep_step_plan_init.restype = ctypes.c_int
    lib.ep_step_plan_layout_dispatch.argtypes = [p]
    lib.ep_step_plan_layout_dispatch.restype = ctypes.c_int
    lib.ep_step_plan_combine.argtypes = [p]
    lib.ep_step_plan_combine.restype = ctypes.c_int
    lib.ep_dispatch_backward.argtypes = [p, p, i64, i32, i32, p, p]
    lib.ep_dispatch_backward.restype = ctypes.c_int
    lib.ep_combine_backward.argtypes = [p, p, p, p, i64, i32, i32, p, p, p]
    lib.ep_combine_backward.restype = ctypes.c_int
    lib.ep_cast_fp8_e4m3.argtypes = [p, p, i64, p]
    lib.ep_cast_fp8_e4m3.restype = ctypes.c_int
    return lib


LIB = _load()


def check(fn, status):
    if status != EP_OK:
        raise EpError(fn, status, LIB)
