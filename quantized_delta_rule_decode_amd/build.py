"""Build libqdr.so (HIP kernels for gfx950 + host runtime) in the package directory.

Each translation unit (one per whole-head storage kind, the row-unit kernels,
the dispatch and the host runtime) compiles to an object in parallel; the
objects are then linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqdr.so")
OBJ = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -ffp-contract=off: only the fused multiply-adds written in the source exist
# (the arithmetic must match the written specification bit for bit).
# The packed-FP32 feature is switched off for every HIP translation unit.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-rdc",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
SOURCES = ["qdr_head_int_step.hip", "qdr_head_int_pack.hip", "qdr_head_int_unpack.hip",
           "qdr_head_int_reset.hip", "qdr_head_int_readout.hip", "qdr_head_int_step_bf16.hip", "qdr_head_int_writeback.hip", "qdr_head_fp16.hip", "qdr_head_fp32.hip", "qdr_rows.hip", "qdr_dispatch.cpp",
           "qdr_runtime.cpp", "qdr_clock.hip"]
# every file the device code is built from (a change to any of them changes the kernels)
# (the clock probe is a diagnostic kernel of its own, not part of the step)
DEVICE_SOURCES = ["qdr_device.h", "qdr_internal.h"] + [s for s in SOURCES
                                                      if s.endswith(".hip") and s != "qdr_clock.hip"]


def device_source_hash() -> str:
    """First 16 hex digits of the sha256 over every device source, in order:
    identifies the kernels that a stored profile was taken from."""
    import hashlib
    h = hashlib.sha256()
    for name in DEVICE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _clean(text: str) -> str:
    return "\n".join(line for line in text.splitlines() if "packed-fp32-ops" not in line)


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(HERE, "..", "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({r.returncode}):\n{_clean(r.stdout + r.stderr)}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_clean(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
