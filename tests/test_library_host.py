"""Host-only checks of libar.so: it loads, exports every entry point the
header declares, and its schedule accounting (ar_plan_bytes, computed by
walking the kernels' own task decoder) agrees with the oracle's independent
tally of the same schedules.  No device calls."""

import os
import re

import numpy as np
import pytest

from all_reduce_reduction_rank_amd import binding
from oracle import traffic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.library()
    names = _declared()
    assert len(names) >= 11
    assert set(names) == set(binding.SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = binding.library()
    for code in range(8):
        assert lib.ar_status_string(code)
    assert lib.ar_status_string(6).decode().startswith("a rank program timed out")


def test_plan_rejects_bad_arguments():
    with pytest.raises(binding.ARError):
        binding.plan_bytes(9, "allreduce", 100, "f32", "ring", "simple")
    with pytest.raises(binding.ARError):
        binding.plan_bytes(0, "allreduce", 100, "f32", "ring", "simple")


CASES = []
_rng = np.random.default_rng(1234)
for _ in range(300):
    n = int(_rng.integers(1, 9))
    op = str(_rng.choice(["allreduce", "reduce_scatter", "allgather"]))
    algo = str(_rng.choice(["oneshot", "twoshot", "ring"]))
    proto = str(_rng.choice(["simple", "ll", "ll128"]))
    dt = str(_rng.choice(["f32", "bf16", "i32"]))
    count = int(_rng.choice([0, 1, 2, 7, 64, 999, 4096, 12345, 70001, 400000]))
    chunk = int(_rng.choice([0, 16, 240, 4096, 100000, 1 << 20]))
    in_place = bool(op == "allreduce" and _rng.integers(0, 2))
    CASES.append((n, op, algo, proto, dt, count, chunk, in_place))


@pytest.mark.parametrize("n,op,algo,proto,dt,count,chunk,in_place", CASES)
def test_plan_bytes_match_oracle_tally(n, op, algo, proto, dt, count, chunk, in_place):
    got = binding.plan_bytes(n, op, count, dt, algo, proto, chunk_bytes=chunk, in_place=in_place)
    want = traffic.tally(op, algo, proto, n, count, dt, in_place=in_place)
    assert got["read"] == want.read
    assert got["write"] == want.write
    assert got["link"] == want.link[:n] or n == 1


def test_headline_plan_bytes():
    # 256 MiB fp32 per rank, N=8, ring, Simple: 5(N-1) S bytes of HBM traffic
    # and 2(N-1)/N S link bytes per rank.
    s = 256 << 20
    p = binding.plan_bytes(8, "allreduce", s // 4, "f32", "ring", "simple", chunk_bytes=512 << 10)
    assert p["hbm"] == 35 * s
    assert p["link"] == [2 * 7 * s // 8] * 8


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("count", [0, 1, 7, 999, 70001])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tree_plan_bytes_match_oracle_tally(n, count, dt):
    got = binding.plan_bytes(n, "allreduce", count, dt, "tree", "simple")
    want = traffic.tally("allreduce", "tree", "simple", n, count, dt)
    assert (got["read"], got["write"]) == (want.read, want.write)
    assert got["link"] == want.link[:n] or n == 1


def test_tree_is_all_reduce_with_simple_only():
    for op, proto in (("allreduce", "ll"), ("allreduce", "ll128"), ("reduce_scatter", "simple"),
                      ("allgather", "simple")):
        with pytest.raises(binding.ARError):
            binding.plan_bytes(4, op, 1000, "f32", "tree", proto)
