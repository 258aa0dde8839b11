"""GPU parity across the message-size sweep above the sizes compared in full.

The sweep of "Collective communication: NCCL's algorithms and protocols, and
custom all-reduce", section "Reading nccl-tests" (`-b 8 -e 1G`), runs every
algorithm and protocol at every size and rank count; tile sizes, ticket lags
and line tiles change with N and with the message size, so each regime is
checked against the oracle here, at sampled positions of full-size calls
(tests/sampled.py).  Inputs are N(0, 1), drawn on the GPU from a seeded
generator.
"""

import pytest
import torch

from all_reduce_reduction_rank_amd import Comm, inputs
from tests.sampled import check_allgather_at, check_allreduce_at, check_reduce_scatter_at, say

pytestmark = pytest.mark.gpu

ESIZE = {"f32": 4, "bf16": 2}
ALGOS = ("oneshot", "twoshot", "ring")
PROTOS = ("simple", "ll", "ll128")


def _release(*bufs):
    for b in bufs:
        del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _allreduce_all(n, count, dt, combos, seed, cfg=60):
    """One set of inputs and one communicator; every (algo, proto) in turn."""
    es = ESIZE[dt]
    send = inputs.device_rank_inputs(n, count, dt, "normal", seed=seed, cfg=cfg)
    recv = [torch.empty_like(t) for t in send]
    lines = any(p != "simple" for _, p in combos)
    c = Comm(n, count * es, count * es if lines else 0)
    try:
        for algo, proto in combos:
            what = f"allreduce {algo}/{proto} {dt} N={n} {count * es} B"
            say(what)
            for t in recv:
                t.view(torch.uint8).fill_(0xA5)
            c.allreduce(send, recv, algo=algo, proto=proto)
            torch.cuda.synchronize()
            assert c.check()[0] == "AR_OK", what
            check_allreduce_at(send, recv, n, count, dt, algo, what, seed=seed)
    finally:
        c.close()
        _release(send, recv)


# N=2 and N=4 above the sizes compared in full: every algorithm (the tree
# with Simple) and protocol, both payload types.
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mib", [2, 32, 512])
@pytest.mark.parametrize("n", [2, 4])
def test_allreduce_n2_n4_sampled(n, mib, dt):
    combos = [(a, p) for a in ALGOS for p in PROTOS] + [("tree", "simple")]
    _allreduce_all(n, (mib << 20) // ESIZE[dt], dt, combos, seed=mib)


# N=8 bf16 with the line protocols at a mid and a large size.
@pytest.mark.parametrize("mib", [8, 128])
def test_allreduce_bf16_line_protocols_sampled(mib):
    combos = [(a, p) for a in ALGOS for p in ("ll", "ll128")]
    _allreduce_all(8, (mib << 20) // 2, "bf16", combos, seed=mib + 1)


# The sweep's largest size with the line protocols, every algorithm.
@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_allreduce_one_gib_line_protocols_sampled(proto):
    _allreduce_all(8, (1 << 30) // 4, "f32", [(a, proto) for a in ALGOS], seed=37)


# Reduce-scatter and all-gather at every rank count, payload type and
# protocol, with the direct and the ring schedule: S = 32 MiB per rank (the
# full buffer: a reduce-scatter sends S and keeps S/N, an all-gather
# receives S).
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_reduce_scatter_and_allgather_32mib_sampled(n, dt):
    es = ESIZE[dt]
    full = (32 << 20) // es
    shard = full // n
    send = inputs.device_rank_inputs(n, full, dt, "normal", seed=n, cfg=61)
    recv = [torch.empty(full, dtype=send[0].dtype, device="cuda") for _ in range(n)]
    c = Comm(n, full * es, full * es)
    try:
        for algo in ("oneshot", "ring"):
            for proto in PROTOS:
                what = f"reduce_scatter {algo}/{proto} {dt} N={n} 32 MiB"
                say(what)
                out = [t[:shard] for t in recv]
                c.reduce_scatter(send, out, algo=algo, proto=proto)
                torch.cuda.synchronize()
                assert c.check()[0] == "AR_OK", what
                check_reduce_scatter_at(send, out, n, shard, dt, algo, what, seed=n)
                what = f"allgather {algo}/{proto} {dt} N={n} 32 MiB"
                say(what)
                src = [t[:shard] for t in send]
                c.allgather(src, recv, algo=algo, proto=proto)
                torch.cuda.synchronize()
                assert c.check()[0] == "AR_OK", what
                check_allgather_at(src, recv, n, shard, dt, algo, what, seed=n)
    finally:
        c.close()
        _release(send, recv)
