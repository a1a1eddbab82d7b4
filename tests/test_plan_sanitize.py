"""The host-side planner and validator built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no GPU code), run over a grid of valid,
invalid and edge-of-range problems (tests/plan_sanitize.cpp).  Any undefined
behaviour or bad access aborts the driver with the sanitizer's report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_09_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_sanitize")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(ROOT, "tests", "plan_sanitize.cpp"), os.path.join(CSRC, "moe_plan.cpp"),
         "-o", exe], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    # verify_asan_link_order=0: the sanitizer runtime need not be the first
    # library of the process (the environment may preload others)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
    assert "0 failed checks" in run.stdout
