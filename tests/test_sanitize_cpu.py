"""The host-side planner and size checks (csrc/plan.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven over every
workload shape (M = 0..513, the configured K and N plus edge sizes, all
three planning dtypes, six CU counts) and a grid of about 7e7 caller-made
plans, valid and not (tests/sanitize/plan_driver.cpp).  Any sanitizer
report aborts the driver; it also checks that completing a planner output
returns it unchanged.  CPU only: the planner makes no HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "latency_skinny_gemm_amd", "csrc"),
           os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
           os.path.join(ROOT, "latency_skinny_gemm_amd", "csrc", "plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "round-trip mismatches 0" in r.stdout, r.stdout
    assert "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stderr
