"""AddressSanitizer + UndefinedBehaviorSanitizer runs of host code (CPU
only): the CPU oracle, and the C ABI's host logic (argument checks,
workspace sizing, group and layer tables, byte accounting) with the kernel
launchers replaced by descriptor-checking stubs.  Both drivers live in
tests/sanitize/ and are built with g++; any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(tmp_path, name, sources, extra):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, *extra, *sources, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_driver",
                         [os.path.join(HERE, "oracle_driver.cpp"),
                          os.path.join(ROOT, "oracle", "moe_oracle.cpp")],
                         ["-pthread", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle")])
    assert "0 failed checks" in out


def test_abi_host_logic_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    csrc = os.path.join(ROOT, "speculative_decode_verify_gate_amd", "csrc")
    out = _build_and_run(tmp_path, "abi_driver",
                         [os.path.join(HERE, "abi_driver.cpp"), os.path.join(csrc, "abi.cpp")],
                         ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                          "-I", os.path.join(ROOT, "include"), "-I", csrc,
                          "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                          "-Wl,-rpath," + os.path.join(rocm, "lib")])
    assert "0 failed checks" in out
