"""Ticket order of every schedule (host only): compiles
tests/schedule_order_check.cpp against the library's planning headers with
g++ and runs it.  Every task a task waits on must have a smaller ticket (the
kernels' deadlock freedom rests on it), and every task must appear once."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_dependency_has_a_smaller_ticket(tmp_path):
    exe = tmp_path / "schedule_order_check"
    src = os.path.join(ROOT, "tests", "schedule_order_check.cpp")
    res = subprocess.run(["g++", "-O2", "-std=c++17", src, "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 bad" in run.stdout
