"""Build libep.so (the C-ABI library) in-tree with hipcc for gfx950.

    python combine_ep_dispatch_amd/build.py

(Run it as a file, not as a package module: importing the package loads
libep.so, which is what this script produces.)

Each .hip file is compiled to an object in parallel, then linked.  The
library links against the HIP runtime that torch loads (torch/lib), so a
process that uses torch for device memory and streams and this library for
the kernels holds one HIP runtime, not two.  Without torch it links
$ROCM_PATH/lib's runtime; EP_HIP_LIB_DIR picks another directory.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libep.so")
SOURCES = ["ep_api.hip", "layout.hip", "layout_dispatch.hip", "dispatch.hip", "fused.hip", "combine.hip",
           "combine_backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # IEEE semantics the kernels' exactness relies on: no contraction of
    # separate multiply/add, correctly rounded binary32 division, binary32
    # denormals kept.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # keep the compiler from forming packed-FP32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hip_lib_dir():
    """Directory of the libamdhip64 to link: $EP_HIP_LIB_DIR if set; else
    the one torch loads (torch/lib), so that a process using torch for
    memory and streams holds a single HIP runtime; else $ROCM_PATH/lib (a
    build for plain C callers on a machine without torch)."""
    import importlib.util

    if os.environ.get("EP_HIP_LIB_DIR"):
        return os.environ["EP_HIP_LIB_DIR"]
    spec = importlib.util.find_spec("torch")
    if spec is not None and spec.submodule_search_locations:
        tl = os.path.join(list(spec.submodule_search_locations)[0], "lib")
        if os.path.exists(os.path.join(tl, "libamdhip64.so")):
            return tl
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln]
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    return "\n".join(lines)


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for log in ex.map(_run, jobs):
            if verbose and log.strip():
                print(log)
    tl = _hip_lib_dir()
    tmp = OUT + ".tmp"
    log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-L" + tl, "-Wl,-rpath," + tl,
                "-lamdhip64", "-o", tmp])
    if verbose and log.strip():
        print(log)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
