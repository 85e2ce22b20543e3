"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code.

Two native drivers under tests/native/ are compiled with g++/gcc under
-fsanitize=address,undefined (host code only: nothing here is built for or
run on a GPU) and must finish cleanly:
  * oracle_sanitize.c drives every entry point of the CPU oracle over pools
    of every kind, unit, gate, scale mode, factor width and refit option,
    on one thread and on three;
  * runtime_sanitize.cpp drives the host-only paths of the library's C ABI
    (descriptor checks, pool layout, argument checks, pool creation without
    a visible device), with the device launches stubbed out.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    rc, out = _run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread",
                    os.path.join(ROOT, "oracle", "qdr_oracle.c"), os.path.join(NATIVE, "oracle_sanitize.c"),
                    "-o", exe, "-lm"])
    assert rc == 0, out
    rc, out = _run([exe])
    assert rc == 0 and out.startswith("ok "), out
    assert "ERROR" not in out and "runtime error" not in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="g++ or the HIP runtime library is not available")
def test_host_runtime_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "runtime_sanitize")
    rc, out = _run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "quantized_delta_rule_decode_amd", "csrc", "qdr_runtime.cpp"),
                    os.path.join(NATIVE, "runtime_sanitize.cpp"), "-o", exe,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert rc == 0, out
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    rc, out = _run([exe], env=env)
    assert rc == 0 and out.startswith("ok "), out
    assert "ERROR" not in out and "runtime error" not in out, out
