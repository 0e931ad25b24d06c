"""The host solver (calibration, water-filling, Lloyd-Max tables, the joint split, token tiers)
built from its C++ sources with AddressSanitizer and UndefinedBehaviorSanitizer, and driven
through every host entry point over ordinary and error inputs (tests/sanitize/host_driver.cpp).
A sanitizer report fails the run.  CPU only: the host sources need no HIP."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "compressed_decode_attention_head_amd", "csrc")
SOURCES = [os.path.join(HERE, "sanitize", "host_driver.cpp"),
           os.path.join(CSRC, "aatc_host.cpp"), os.path.join(CSRC, "aatc_tiers.cpp")]


def test_host_solver_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "host_driver")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    r = subprocess.run([cxx] + flags + SOURCES + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "all checks passed" in r.stdout
