"""The host half of libfp8pa (planner and argument checks, csrc/host.cpp)
built with AddressSanitizer and UndefinedBehaviorSanitizer and run on the
CPU over a grid of shapes and a seeded fuzz of every shape field
(tests/host_plan_check.cpp).  Any sanitizer report or broken plan invariant
fails the run.  No GPU: host.cpp includes no HIP header.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planner_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++") or shutil.which("clang++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_plan_check")
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", f"-I{ROOT}/include"]
    src = [os.path.join(ROOT, "decode_attention_paged_fp8pa_amd", "csrc", "host.cpp"),
           os.path.join(ROOT, "tests", "host_plan_check.cpp")]
    r = subprocess.run([cxx, *flags, *src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:] + r.stderr[-6000:])
    assert "0 failures" in r.stdout
