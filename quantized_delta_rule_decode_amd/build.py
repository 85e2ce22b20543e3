"""Build libqdr.so (HIP kernels for gfx950 + host runtime) in the package directory."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqdr.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: only the fused multiply-adds written in the source exist
# (the arithmetic must match the written specification bit for bit).
# The packed-FP32 feature is switched off for every HIP translation unit.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-rdc",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
SOURCES = ["qdr_kernels.hip", "qdr_runtime.cpp"]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
