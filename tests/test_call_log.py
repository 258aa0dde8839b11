"""The communicator's call log and AR_DEBUG line (host only): compiles
tests/call_log_check.cpp against the library's log header with g++ and runs
it."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_call_log_keeps_the_last_calls_in_order(tmp_path):
    exe = tmp_path / "call_log_check"
    src = os.path.join(ROOT, "tests", "call_log_check.cpp")
    res = subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", src, "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 bad" in run.stdout
