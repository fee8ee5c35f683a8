"""The host planner and the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

tests/sanitize/abi_driver.cpp drives every host-side path of the ABI over
seeded random batches (plan, run, paged and FP8 runs, the one-shot plan and
workspace caches across 11 streams, shared prefix, state merges, invalid
arguments, injected allocation failures) against tests/sanitize/
host_device_stub.cpp, which replaces the HIP runtime by host memory and the
kernel launches by walks that touch every byte range the kernels would read
or write.  A report from either sanitizer, a broken launch contract or a
wrong status fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "varlen_prefill_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(HERE, "_build")


def _build() -> str:
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", SRC,
           os.path.join(SRC, "rp_plan.cpp"), os.path.join(SRC, "rp_api.cpp"),
           os.path.join(HERE, "host_device_stub.cpp"), os.path.join(HERE, "abi_driver.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def test_planner_and_abi_under_sanitizers():
    exe = _build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env.pop("RP_FAULT_INJECT", None)
    res = subprocess.run([exe, "200"], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "abi driver: ok" in res.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
