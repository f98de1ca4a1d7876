"""The oracle and the library's host runtime under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Both are built with gcc / g++ (host code only; no GPU code is involved):
  - oracle/rr_oracle.c with tests/sanitize/oracle_driver.c, which calls every
    oracle entry point on small seeded shapes (whole and ragged lengths,
    causal and not, G = 1 and G > 1, tau < 1 and tau = 1, row masks,
    thresholds per head, sampled rows, a decode step);
  - csrc/rr_host.cpp (argument checks, workspace layout, varlen and decode
    sequencing) with tests/sanitize/host_stubs.cpp in place of the kernel
    launches and tests/sanitize/host_driver.cpp, which calls every C-ABI
    entry point; the stand-ins check that every buffer carved out of a
    workspace lies inside it.
Any sanitizer report aborts the program (-fno-sanitize-recover=all).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no gcc")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
                           os.path.join(ROOT, "oracle", "rr_oracle.c"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
    assert "oracle driver ok" in _run(exe)


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="HIP headers not installed")
def test_host_runtime_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "dynamic_block_sparse_rr_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                           "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(csrc, "rr_host.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe])
    assert "host driver ok" in _run(exe)
