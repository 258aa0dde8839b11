"""Tile choice of the schedules that never wait (host only): compiles
tests/tile_rule_check.cpp against the library's planning header with g++ and
runs it.  Such calls launch without the ticket counter when one grid covers
their tasks, and the planner grows their tiles toward that within a bound.
It also checks the placement of a one-shot's tile programs on one die
(die_ticket): every ticket exactly once, each tile's programs on one die."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_never_waiting_calls_fit_one_grid_when_a_bounded_tile_allows(tmp_path):
    exe = tmp_path / "tile_rule_check"
    src = os.path.join(ROOT, "tests", "tile_rule_check.cpp")
    res = subprocess.run(["g++", "-O2", "-std=c++17", src, "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert " 0 bad" in run.stdout
    grown = int(run.stdout.split(" grown")[0].split(",")[-1])
    assert grown > 0  # the rule is exercised
    assert " 560 placements" in run.stdout  # die_ticket checked for G = 1..8, 1..70 groups
