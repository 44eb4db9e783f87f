"""The host planner (csrc/plan.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, host code only (no HIP: the three device hooks are stubbed in
tests/host_asan/plan_driver.cpp), and run over random iterations, the pages' workload
shapes (including the 128K-context metadata of 524,288 block-table entries) and refused
metadata.  The driver checks every plan's work lists itself; the run must end with status
0 and no sanitizer report (leaks included)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "varlen_paged_attention_amd", "csrc"),
           os.path.join(ROOT, "varlen_paged_attention_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "host_asan", "plan_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert "0 failures" in run.stdout
