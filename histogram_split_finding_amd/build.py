"""Builds libgbdt_hip.so (the C-ABI library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgbdt_hip.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["gbdt_kernels.hip", "gbdt_driver.hip", "gbdt_predict.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: FP64 gain / weight / prediction arithmetic is evaluated
# one IEEE operation at a time, as on the CPU.  The packed-FP32 target
# feature is switched off for all device code.  Kernel arguments are
# preloaded into SGPRs at wave launch (the first 16 dwords), which saves the
# kernels' first scalar round trip; without firmware support the code object's
# own prologue loads them instead.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    print(LIB_PATH)
    sys.exit(0)
