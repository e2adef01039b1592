"""The library's host half and the C oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (g++ / gcc, CPU only), each driven by a randomised
program in tests/sanitize/: memory errors, leaks and undefined behaviour abort
that program.  host.cpp is the library's own source file; its three HIP runtime
calls are stubbed by the test program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs g++ and gcc")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    return res.stdout


def test_host_half_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "segmented_gather_gemm_segments_amd", "csrc"),
                           os.path.join(ROOT, "segmented_gather_gemm_segments_amd", "csrc", "host.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe])
    assert "host driver ok" in _run(exe)


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
                           os.path.join(ROOT, "oracle", "sgmv_oracle.c"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe])
    assert "oracle driver ok" in _run(exe)
