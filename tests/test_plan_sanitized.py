"""The workspace planner (plan.h, pure host arithmetic) built with the address
and undefined-behaviour sanitizers and run over a sweep of shapes: chunks and
trunks cover heads and tokens exactly, workspace regions are aligned, inside
the total and disjoint, and bad shapes are refused (tests/native/plan_check.cpp)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    src = os.path.join(HERE, "native", "plan_check.cpp")
    inc = os.path.join(ROOT, "head_chunked_context_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", inc, src, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "failures: 0" in r.stdout
