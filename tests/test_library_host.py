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


def test_noalloc_argument_errors_need_no_device():
    # Argument checks come before any HIP call: these run without a GPU.
    import ctypes
    lib = binding.library()
    P = ctypes.c_void_p
    ptrs = (P * 8)(*[0x10000 * (i + 1) for i in range(8)])
    outs = (P * 8)(*[0x10000000 * (i + 1) for i in range(8)])
    st = lambda n, count, dt=0, algo=2, proto=0, s=ptrs, r=outs: lib.ar_allreduce_noalloc(  # noqa: E731
        n, s, r, count, dt, algo, proto, 0, None)
    assert st(9, 16) == 1 and st(0, 16) == 1                  # AR_ERR_INVALID: rank count
    assert st(8, 16, proto=1) == 2 and st(8, 16, proto=2) == 2  # LL / LL128: AR_ERR_UNSUPPORTED
    assert st(8, (1 << 28) + 1) == 4                          # fp32 above 1 GiB per rank: AR_ERR_TOO_LARGE
    assert st(8, (1 << 29) + 4, dt=1) == 4                    # bf16 likewise
    assert st(8, 0) == 0                                      # count 0: nothing to do
    assert st(8, 16, algo=5) == 1 and st(8, 16, dt=3) == 1    # bad enums
    assert st(2, 16, s=None) == 1                             # null pointer array
    odd = (P * 8)(*[0x10000 * (i + 1) + 4 for i in range(8)])
    assert st(4, 16, s=odd) == 1                              # misaligned rank buffer


def test_noalloc_device_array_holds_every_schedule_up_to_one_gib():
    # On a host with no GPU a call that passes every argument and capacity
    # check stops at the first HIP call (AR_ERR_HIP); one whose flags would
    # not fit the device array stops earlier with AR_ERR_TOO_LARGE.  Every
    # schedule, in and out of place, must fit at the 1 GiB limit.
    import ctypes

    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("needs a host without a GPU: the fake pointers below must never reach a kernel")
    lib = binding.library()
    P = ctypes.c_void_p
    for n in range(2, 9):
        ptrs = (P * n)(*[(1 << 40) * (i + 1) for i in range(n)])
        outs = (P * n)(*[(1 << 40) * (i + 1) + (1 << 39) for i in range(n)])
        for algo in range(5):
            for dt, es in ((0, 4), (1, 2)):
                count = (1 << 30) // es
                for recv in (outs, ptrs):  # out of place, in place
                    st = lib.ar_allreduce_noalloc(n, ptrs, recv, count, dt, algo, 0, 0, None)
                    assert st == 5, (n, algo, dt, recv is ptrs, st)


def test_stream_ceiling_argument_errors_need_no_device():
    import ctypes
    lib = binding.library()
    P = ctypes.c_void_p
    bufs = (P * 8)(*[0x100000 * (i + 1) for i in range(8)])
    outs = (P * 2)(*[0x10000000 * (i + 1) for i in range(2)])
    st = lambda r, w, nbytes, flags=0, unroll=8, per_cu=0, sink=None: lib.ar_stream_ceiling(  # noqa: E731
        r, bufs, w, outs, nbytes, sink, flags, unroll, per_cu, None)
    assert st(9, 1, 4096) == 1 and st(1, 3, 4096) == 1 and st(0, 0, 4096) == 1   # stream counts
    assert st(1, 1, 4100) == 1 and st(1, 1, (2 << 30) + 16) == 1                  # size
    assert st(1, 1, 4096, flags=4) == 1 and st(1, 1, 4096, unroll=5) == 1        # flags, unroll
    assert st(1, 1, 4096, per_cu=-1) == 1
    assert st(1, 0, 4096) == 1                                                    # read-only needs a sink
