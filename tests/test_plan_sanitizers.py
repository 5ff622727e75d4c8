"""The host planner (csrc/plan.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, g++) and driven by
tests/native/plan_fuzz.cpp: random and nested block tables, the 64-group and
512-request-order limits, autotune records and every validation error path.
Any memory or undefined-behaviour error aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "shared_prefix_attention_amd", "csrc"),
           os.path.join(ROOT, "shared_prefix_attention_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
