"""Host sanitizer runs (CPU tier): the float64 oracle and the library's host
code built with AddressSanitizer + UndefinedBehaviorSanitizer (gcc / g++,
host code only) and driven over seeded random shapes by the drivers in
tests/sanitize/.  Any out-of-bounds access, leak or undefined arithmetic
aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    if r.returncode != 0 and "sanitize" in r.stderr and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-pthread", "oracle/oracle.c",
                "tests/sanitize/oracle_driver.c", "-o", exe, "-lm"], exe, tmp_path)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_library_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                "-Iinclude", "-Ipaged_gqa_kv_decode_amd/csrc",
                "paged_gqa_kv_decode_amd/csrc/vk_host.cpp", "tests/sanitize/host_driver.cpp",
                "-o", exe], exe, tmp_path)
    assert " 0 failures" in out
