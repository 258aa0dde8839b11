"""ar_allreduce_noalloc (the all-reduce that allocates nothing) against
ar_allreduce on a communicator: the same schedules on the same kernels must
give the same bits.  Each case makes two calls in a row, the second on a
smaller input, so the second runs on the device array as the first left it.
"""

import sys

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import Comm, allreduce_noalloc, inputs
from oracle import collectives as C
from tests.gpu_util import assert_same, to_host

pytestmark = pytest.mark.gpu

ESIZE = {"f32": 4, "bf16": 2, "i32": 4}
DIST = {"f32": "normal", "bf16": "normal", "i32": "int20"}


def _say(*what):
    print("CASE", *what, flush=True, file=sys.stderr)


def _pair(n, count, dt, algo, seed, in_place=False):
    """(noalloc outputs, communicator outputs, inputs) of one call."""
    send = inputs.device_rank_inputs(n, count, dt, DIST[dt], seed=seed, cfg=70)
    ref_in = [t.clone() for t in send]
    comm = Comm(n, count * ESIZE[dt], 0)
    want = comm.allreduce(ref_in, None if in_place else [torch.empty_like(t) for t in send], algo=algo)
    torch.cuda.synchronize()
    assert comm.check()[0] == "AR_OK"
    comm.close()
    if in_place:
        got = allreduce_noalloc(send, None, algo=algo)
    else:
        got = allreduce_noalloc(send, [torch.empty_like(t).fill_(7) for t in send], algo=algo)
    torch.cuda.synchronize()
    return got, want, ref_in if not in_place else None


@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("algo", ["oneshot", "twoshot", "ring", "tree", "auto"])
def test_noalloc_matches_allreduce_twice_second_smaller(algo, dt):
    n = 8
    for count, seed in ((3 * (1 << 20) + 17, 1), (4099, 2)):  # second call: smaller (and ragged)
        _say("noalloc", algo, dt, n, count)
        got, want, _ = _pair(n, count, dt, algo, seed)
        for r in range(n):
            assert_same(to_host(got[r], dt), to_host(want[r], dt), f"noalloc {algo} {dt} N={n} count={count} rank {r}")


@pytest.mark.parametrize("n", [1, 2, 5])
def test_noalloc_small_rank_counts_and_the_oracle(n):
    dt = "f32"
    for count in (40961, 77):
        _say("noalloc-oracle", n, count)
        host = inputs.rank_inputs(n, count, dt, "normal", seed=count, cfg=71)
        send = [torch.from_numpy(x).cuda() for x in host]
        for algo in ("oneshot", "twoshot", "ring"):
            recv = allreduce_noalloc(send, [torch.empty_like(t) for t in send], algo=algo)
            torch.cuda.synchronize()
            want = C.allreduce(host, dt, algo)
            for r in range(n):
                assert_same(recv[r].cpu().numpy(), want[r], f"noalloc {algo} N={n} count={count} rank {r}")


@pytest.mark.parametrize("algo", ["oneshot", "twoshot", "ring"])
def test_noalloc_in_place_twice_second_smaller(algo):
    n, dt = 4, "bf16"
    for count, seed in ((1 << 20, 3), (1000, 4)):
        _say("noalloc-in-place", algo, count)
        got, want, _ = _pair(n, count, dt, algo, seed, in_place=True)
        for r in range(n):
            assert_same(to_host(got[r], dt), to_host(want[r], dt), f"noalloc in place {algo} count={count} rank {r}")


def test_noalloc_large_two_shot_then_small_ring():
    # A 64 MiB two-shot (tiles of 64 KiB, a ticket lag) then a small ring.
    n, dt = 8, "f32"
    for count, algo, seed in (((64 << 20) // 4, "twoshot", 5), (12345, "ring", 6)):
        _say("noalloc-large", algo, count)
        got, want, _ = _pair(n, count, dt, algo, seed)
        for r in range(n):
            g, w = to_host(got[r], dt), to_host(want[r], dt)
            assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"noalloc {algo} count={count} rank {r}"
