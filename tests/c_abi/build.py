"""Build the C-ABI test driver tests/c_abi/ep_step from ep_step.c with gcc
(plain C plus the HIP runtime; links libep.so, found next to the package at
run time through an $ORIGIN-relative rpath).  Run as a file after the
library is built: python tests/c_abi/build.py"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
OUT = os.path.join(HERE, "ep_step")


def command(out=OUT):
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
            os.path.join(HERE, "ep_step.c"), "-o", out,
            "-L", os.path.join(ROOT, "combine_ep_dispatch_amd"), "-lep",
            "-Wl,-rpath,$ORIGIN/../../combine_ep_dispatch_amd",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def main():
    subprocess.run(command(), check=True)
    print(OUT)


if __name__ == "__main__":
    sys.exit(main())
