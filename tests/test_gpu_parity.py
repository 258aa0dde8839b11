"""GPU parity: every collective x algorithm x protocol x payload type, through
the C ABI (libar.so via the ctypes binding), compared element by element
with the CPU oracle on the same seeded inputs.  Integer and same-order
floating point results must be bit-exact."""

import sys

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import ARError, Comm, inputs
from oracle import collectives as C
from tests.gpu_util import assert_same, empty, to_dev, to_host

pytestmark = pytest.mark.gpu

ALGOS = ("oneshot", "twoshot", "ring")
PROTOS = ("simple", "ll", "ll128")
DTYPES = ("f32", "bf16", "i32")
MAX_BYTES = 64 << 20
LINE_BYTES = 16 << 20

_COMMS = {}


def comm(n):
    if n not in _COMMS:
        _COMMS[n] = Comm(n, MAX_BYTES, LINE_BYTES)
    return _COMMS[n]


def _dist(dt):
    return "int20" if dt == "i32" else "normal"


def _say(*what):
    print("CASE", *what, flush=True, file=sys.stderr)


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 8])
def test_many_pass_colocated_line_one_shot(dt, n, proto):
    # Line one-shots of several passes per workgroup (LL: 4 KiB passes, up
    # to 8; LL128: 128-line passes of 15 KiB, up to 2), a ragged tail, out
    # of place and in place, all without the ticket counter and equal to the
    # oracle.
    es = 2 if dt == "bf16" else 4
    tiles = 256 // n
    pass_bytes, cases = (4096, ((5, 0), (8, 0), (5, 3))) if proto == "ll" else (15360, ((2, 0), (2, 3)))
    c = Comm(n, tiles * pass_bytes * 8, tiles * pass_bytes * 8 * 4)
    for passes, tail in cases:
        count = tiles * passes * pass_bytes // es - tail
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=passes + tail, cfg=82)
        want = C.allreduce(host, dt, "oneshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("coloc many-pass", proto, dt, n, passes, count)
        c.allreduce(send, recv, algo="oneshot", proto=proto)
        torch.cuda.synchronize()
        assert c.debug_calls(1)[0]["counter_free"] == 1, (dt, n, passes, count)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"coloc many-pass {proto} {dt} N={n} count={count} rank {r}")
        c.allreduce(send, None, algo="oneshot", proto=proto)
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(send[r], dt), want[r], f"coloc many-pass in place {proto} {dt} N={n} count={count} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 8])
def test_colocated_ll128_two_shot(dt, n):
    # Two-shot LL128 with one workgroup per (tile, rank): tiles of 1 and 2
    # passes, a ragged count, out of place and in place; bf16 also with odd
    # counts (loads and stores then go element by element, in a kernel that
    # fits one workgroup per CU, so these grids stay within half of that:
    # 128).  All without the ticket counter, equal to the oracle.
    es = 2 if dt == "bf16" else 4
    c = Comm(n, 2 << 20 << 3, 2 << 20 << 4)
    cases = [(1, 0, 256), (2, 0, 256), (2, 4, 256)]
    if dt == "bf16":
        cases += [(1, 1, 128), (1, 3, 128)]
    for passes, tail, grid in cases:
        tiles = grid // n
        count = n * tiles * passes * 15360 // es - tail
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=passes * 10 + tail, cfg=83)
        want = C.allreduce(host, dt, "twoshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("coloc two-shot", dt, n, passes, tail, grid, count)
        c.allreduce(send, recv, algo="twoshot", proto="ll128")
        torch.cuda.synchronize()
        assert c.debug_calls(1)[0]["counter_free"] == 1, (dt, n, passes, count)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"coloc two-shot {dt} N={n} count={count} rank {r}")
        c.allreduce(send, None, algo="twoshot", proto="ll128")
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(send[r], dt), want[r], f"coloc two-shot in place {dt} N={n} count={count} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [3, 5, 8])
def test_one_shot_placed_by_die(dt, n):
    # Simple one-shots whose N inputs exceed one die's 4 MiB L2 run each
    # tile's N rank programs on one die: a grid of 8 N ceil(tiles / 8)
    # workgroups, some of them idle.  Tile counts that are and are not a
    # multiple of 8, ragged counts: every output equals the oracle.
    es = 2 if dt == "bf16" else 4
    c = Comm(n, 8 << 20, 0)
    for rank_bytes, tail in (((4 << 20) // n + (1 << 16), 0), (3 << 20, 5), (8 << 20, 1), ((5 << 20) + 4096, 0)):
        count = rank_bytes // es - tail
        assert n * count * es > 4 << 20
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=rank_bytes % 997 + tail, cfg=87)
        want = C.allreduce(host, dt, "oneshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("one-shot by die", dt, n, count)
        c.allreduce(send, recv, algo="oneshot", proto="simple")
        torch.cuda.synchronize()
        rec = c.debug_calls(1)[0]
        assert rec["counter_free"] == 1 and rec["by_die"] == n and rec["grid"] % (8 * n) == 0, rec
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"one-shot by die {dt} N={n} count={count} rank {r}")
    if n == 3:
        # 510 tasks in one grid, whose placement by die would need 528
        # workgroups: under a budget of 520 the call keeps its 510.
        count = (3 << 20) // es
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=11, cfg=87)
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        c.set_max_workgroups(520)
        c.allreduce(send, recv, algo="oneshot", proto="simple")
        torch.cuda.synchronize()
        rec = c.debug_calls(1)[0]
        assert rec["counter_free"] == 1 and rec["by_die"] == 0 and rec["grid"] <= 520, rec
        want = C.allreduce(host, dt, "oneshot")
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"one-shot budget {dt} rank {r}")
        c.set_max_workgroups(0)
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [3, 8])
def test_one_shot_ticketed_by_die(dt, n):
    # One-shots too large for one grid draw their tickets from one counter
    # per die (each die's share: the tiles whose N programs run there).
    # Default grid, a budget of 12 workgroups (a grid of 8: one per die) and
    # of 5 (fewer than the dies: one shared counter); a ragged count.  Every
    # output equals the oracle, and repeated calls re-arm the counters.
    es = 2 if dt == "bf16" else 4
    c = Comm(n, 48 << 20, 0)
    count = (48 << 20) // es - 7  # 128 KiB tiles: 384 per buffer, beyond one grid
    host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=n, cfg=89)
    want = C.allreduce(host, dt, "oneshot")
    send = [to_dev(x, dt) for x in host]
    for budget in (0, 12, 5, 0):
        c.set_max_workgroups(budget)
        recv = [empty(count, dt) for _ in range(n)]
        _say("one-shot ticketed by die", dt, n, count, budget)
        c.allreduce(send, recv, algo="oneshot", proto="simple")
        torch.cuda.synchronize()
        rec = c.debug_calls(1)[0]
        assert rec["counter_free"] == 0, rec
        assert (rec["by_die"] == n and rec["grid"] % 8 == 0) or (budget == 5 and rec["grid"] < 8), rec
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"one-shot by die {dt} N={n} budget {budget} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_all_gather_placed_by_die(dt, n):
    # Direct all-gathers writing N x S >= 32 MiB run each shard tile's N
    # receivers on one die (a grid of 8 N ceil(groups / 8) workgroups):
    # whole and ragged shards, every output equal to the oracle.
    es = 2 if dt == "bf16" else 4
    c = Comm(n, 32 << 20, 0)
    for full_bytes, tail in (((32 << 20) // n, 0), ((32 << 20) // n + 4096, 3)):
        count = (full_bytes // n) // es - tail  # per-rank send elements
        assert n * n * count * es >= 32 << 20 or tail
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=full_bytes % 991 + tail, cfg=88)
        want = C.allgather(host, dt, "oneshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(n * count, dt) for _ in range(n)]
        _say("all-gather by die", dt, n, count)
        c.allgather(send, recv, algo="oneshot", proto="simple")
        torch.cuda.synchronize()
        rec = c.debug_calls(1)[0]
        assert rec["counter_free"] == 1, rec
        if n * n * count * es >= 32 << 20:
            assert rec["by_die"] == n and rec["grid"] % (8 * n) == 0, rec
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"all-gather by die {dt} N={n} count={count} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_colocated_ll_two_shot(dt, n):
    # Two-shot LL with one workgroup per (tile, rank): blocks just over one
    # 4 KiB pass (a second tile of 32 bytes), tiles of one pass (rounds of 4
    # words a thread), of 3 and of 8 passes (rounds of 8 words, the last one
    # partly past the tile), a ragged count, out of place and in place; bf16
    # also with odd counts (element by element).  All without the ticket
    # counter, equal to the oracle.
    es = 2 if dt == "bf16" else 4
    tiles = 256 // n
    c = Comm(n, 8 << 20, 16 << 20)
    cases = [(n * 4128 // es, 0), (n * tiles * 4096 // es, 0), (n * tiles * 3 * 4096 // es, 4),
             (n * tiles * 8 * 4096 // es, 0), (n * tiles * 8 * 4096 // es - 8, 0)]
    if dt == "bf16":
        cases += [(n * tiles * 4096 // es, 1), (n * tiles * 3 * 4096 // es, 3)]
    for base, tail in cases:
        count = base - tail
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=count % 1000, cfg=86)
        want = C.allreduce(host, dt, "twoshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("coloc ll two-shot", dt, n, count)
        c.allreduce(send, recv, algo="twoshot", proto="ll")
        torch.cuda.synchronize()
        assert c.debug_calls(1)[0]["counter_free"] == 1, (dt, n, count)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"coloc ll two-shot {dt} N={n} count={count} rank {r}")
        c.allreduce(send, None, algo="twoshot", proto="ll")
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(send[r], dt), want[r], f"coloc ll two-shot in place {dt} N={n} count={count} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("proto,n,rank,step", [("ll", 4, 1, 0), ("ll", 8, 6, 1), ("ll128", 4, 2, 0), ("ll128", 8, 3, 1)])
def test_colocated_ll_two_shot_withheld_lines(proto, n, rank, step):
    # One rank program of a colocated LL / LL128 two-shot does not finish its
    # lines of one step (its sends, or its published sum; LL128: payload
    # without the flag words): the receives waiting on them give up at 50 ms
    # and name the first blocked (rank, step) of the oracle's transfer
    # graph; after a reset the same call is exact.
    from oracle import sim

    c = Comm(n, 1 << 20, 1 << 20)
    count = n * (64 << 10) // 4
    host = inputs.rank_inputs(n, count, "f32", "normal", seed=6)
    send = [to_dev(x, "f32") for x in host]
    recv = [empty(count, "f32") for _ in range(n)]
    c.inject(rank, step, timeout_us=50_000)
    _say("inject coloc two-shot", proto, n, rank, step)
    c.allreduce(send, recv, algo="twoshot", proto=proto)
    assert c.debug_calls(1)[0]["counter_free"] == 1
    status, r, s = c.check()
    assert status == "AR_ERR_TIMEOUT"
    _, first = sim.blocked("allreduce", "twoshot", n, withheld=(rank, step), proto=proto)
    assert (r, s) == first
    c.inject(-1, -1)
    c.reset()
    c.allreduce(send, recv, algo="twoshot", proto=proto)
    torch.cuda.synchronize()
    want = C.allreduce(host, "f32", "twoshot")
    for q in range(n):
        assert_same(to_host(recv[q], "f32"), want[q], f"after reset rank {q}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_colocated_simple_two_shot(dt, n):
    # Simple two-shots of 64 KiB to 8 MiB blocks run one workgroup per (tile,
    # rank): results equal the oracle out of place, in place and with ragged
    # counts; a workgroup budget below the grid takes the ticketed schedule.
    es = 2 if dt == "bf16" else 4
    c = Comm(n, 8 << 20, 0)
    for block_bytes, tail in ((64 << 10, 0), (1 << 20, 5), (3 << 20, 0), (8 << 20, 1)):
        count = min(n * block_bytes, 8 << 20) // es - tail
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=block_bytes + tail, cfg=84)
        want = C.allreduce(host, dt, "twoshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("coloc simple two-shot", dt, n, count)
        c.allreduce(send, recv, algo="twoshot", proto="simple")
        torch.cuda.synchronize()
        assert c.debug_calls(1)[0]["counter_free"] == 1, (dt, n, count)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"coloc simple two-shot {dt} N={n} count={count} rank {r}")
        c.allreduce(send, None, algo="twoshot", proto="simple")
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(send[r], dt), want[r], f"coloc simple two-shot in place {dt} N={n} count={count} rank {r}")
    c.set_max_workgroups(n)
    count = n * (256 << 10) // es
    host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=2, cfg=85)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(count, dt) for _ in range(n)]
    c.allreduce(send, recv, algo="twoshot", proto="simple")
    torch.cuda.synchronize()
    assert c.debug_calls(1)[0]["counter_free"] == 0
    want = C.allreduce(host, dt, "twoshot")
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"budget simple two-shot {dt} N={n} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("n,rank,step", [(4, 2, 0), (8, 5, 0)])
def test_colocated_simple_two_shot_withheld_signal(n, rank, step):
    # One rank program of a colocated Simple two-shot skips its fold signal:
    # the gathers waiting on it give up at 50 ms and name the first blocked
    # (rank, step) of the ticketed schedule's model.
    from oracle import sim

    c = Comm(n, 1 << 20, 0)
    count = n * (64 << 10) // 4
    host = inputs.rank_inputs(n, count, "f32", "normal", seed=5)
    send = [to_dev(x, "f32") for x in host]
    recv = [empty(count, "f32") for _ in range(n)]
    c.inject(rank, step, timeout_us=50_000)
    _say("inject coloc two-shot", n, rank, step)
    c.allreduce(send, recv, algo="twoshot")
    assert c.debug_calls(1)[0]["counter_free"] == 1
    status, r, s = c.check()
    assert status == "AR_ERR_TIMEOUT"
    _, first = sim.blocked("allreduce", "twoshot", n, withheld=(rank, step))
    assert (r, s) == first
    c.inject(-1, -1)
    c.reset()
    c.allreduce(send, recv, algo="twoshot")
    torch.cuda.synchronize()
    want = C.allreduce(host, "f32", "twoshot")
    for q in range(n):
        assert_same(to_host(recv[q], "f32"), want[q], f"after reset rank {q}")
    assert c.check()[0] == "AR_OK"
    c.close()


def run_allreduce(n, count, dt, algo, proto, chunk=0, seed=0, in_place=False, dist=None):
    host = inputs.rank_inputs(n, count, dt, dist or _dist(dt), seed=seed, cfg=100 + n)
    send = [to_dev(x, dt) for x in host]
    recv = send if in_place else [empty(count, dt) for _ in range(n)]
    _say("allreduce", n, count, dt, algo, proto, chunk, "inplace" if in_place else "")
    comm(n).allreduce(send, recv, algo=algo, proto=proto, chunk_bytes=chunk)
    torch.cuda.synchronize()
    got = [to_host(t, dt) for t in recv]
    want = C.allreduce(host, dt, algo, chunk_bytes=chunk or C.DEFAULT_CHUNK_BYTES)
    for r in range(n):
        assert_same(got[r], want[r], f"allreduce {algo}/{proto} {dt} N={n} count={count} rank {r}")
    st = comm(n).check()
    assert st[0] == "AR_OK", st


# ---------------------------------------------------------------- all-reduce
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("n", [2, 3, 8])
def test_allreduce_matrix(n, algo, proto, dt):
    # 1 element (blocks mostly empty), a ragged tail, several tiles per block.
    for count in (1, 7, 1000, 70001):
        run_allreduce(n, count, dt, algo, proto, seed=count)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8])
def test_simple_fold_every_rank_count(n, dt):
    # The Simple one-shot and two-shot folds are compiled per term count:
    # every N, with a ragged tail, one pass and many passes per tile.
    for algo in ("oneshot", "twoshot"):
        for count in (5, 4097, 262147):
            run_allreduce(n, count, dt, algo, "simple", seed=count + n)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dt", DTYPES)
def test_ring_many_chunks(proto, dt):
    # Small chunks: many chunk loops per block, short last tiles.
    for chunk in (16, 240, 4096, 100000):
        run_allreduce(4, 5003, dt, "ring", proto, chunk=chunk, seed=chunk)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
def test_allreduce_in_place(algo, proto):
    for dt in DTYPES:
        for n, count in ((2, 4096), (8, 33333)):
            run_allreduce(n, count, dt, algo, proto, seed=7, in_place=True)


@pytest.mark.parametrize("algo", ALGOS)
def test_all_ones_sum_to_n(algo):
    # "NCCL collectives..." sanity test: an all-reduce of ones gives N.
    for n in (2, 5, 8):
        for proto in PROTOS:
            for dt in DTYPES:
                run_allreduce(n, 128, dt, algo, proto, dist="ones")


def test_config_small_n2_4096_f32():
    # N=2, 4096 fp32 uniform[-1,1]: every algorithm and protocol, plus ones.
    for algo in ALGOS:
        for proto in PROTOS:
            run_allreduce(2, 4096, "f32", algo, proto, dist="uniform")
            run_allreduce(2, 4096, "f32", algo, proto, dist="ones")


@pytest.mark.parametrize("algo", ALGOS)
def test_ll_lines_never_meet_ll128_payload(algo):
    # An LL reader takes bytes 4-7 of each 8-byte slot as the line's flag.
    # Each protocol stages in its own region, so an earlier LL128 call's
    # payload can never sit there: here every LL128 payload word equals the
    # flag the next LL call writes, and that LL call must still match the
    # oracle.
    n = 4
    c = Comm(n, 1 << 20, 1 << 20)
    try:
        for count in (4096, 30001, 65536):
            calls = c.debug_state()["calls"]
            # the LL128 call runs with epoch `calls`, the LL call with
            # calls + 1, whose LL flag is calls + 2
            bait = [torch.full((count,), calls + 2, dtype=torch.int32, device="cuda") for _ in range(n)]
            c.allreduce(bait, [empty(count, "i32") for _ in range(n)], algo=algo, proto="ll128")
            host = inputs.rank_inputs(n, count, "i32", "int20", seed=count, cfg=400 + n)
            send = [to_dev(x, "i32") for x in host]
            recv = [empty(count, "i32") for _ in range(n)]
            _say("ll after ll128 bait", algo, n, count)
            c.allreduce(send, recv, algo=algo, proto="ll")
            torch.cuda.synchronize()
            want = C.allreduce(host, "i32", algo)
            for r in range(n):
                assert_same(to_host(recv[r], "i32"), want[r], f"LL {algo} after LL128 bait count={count} rank {r}")
        assert c.check()[0] == "AR_OK"
    finally:
        c.close()


def test_eight_bytes_per_rank():
    # 8 B per rank at N=8: most blocks empty, every LL128 line partial.
    for algo in ALGOS:
        for proto in PROTOS:
            run_allreduce(8, 2, "f32", algo, proto)
            run_allreduce(8, 4, "bf16", algo, proto)


@pytest.mark.parametrize("op,nbytes", [("allreduce", 512 << 10), ("allreduce", 640 << 10),
                                       ("allgather", 512 << 10), ("allgather", 8 << 20),
                                       ("reduce_scatter", 2 << 20)])
def test_mid_size_calls_that_never_wait_skip_the_ticket_counter(op, nbytes):
    # Simple one-shot and direct RS/AG calls of these sizes take tiles that
    # fit one grid, so they launch without the ticket counter: such a call
    # leaves the device call counter where it was.  The results still match
    # the oracle.
    n, dt = 8, "bf16"
    c = Comm(n, nbytes, 0)
    try:
        full = nbytes // 2
        shard = full // n
        host = inputs.rank_inputs(n, shard if op == "allgather" else full, dt, "normal", seed=nbytes, cfg=500)
        send = [to_dev(x, dt) for x in host]
        recv = [empty(full if op != "reduce_scatter" else shard, dt) for _ in range(n)]
        _say("counter-free", op, n, nbytes)
        before = c.debug_state()["calls"]
        if op == "allreduce":
            c.allreduce(send, recv, algo="oneshot", proto="simple")
            want = C.allreduce(host, dt, "oneshot")
        elif op == "allgather":
            c.allgather(send, recv, algo="oneshot", proto="simple")
            want = C.allgather(host, dt, "oneshot")
        else:
            c.reduce_scatter(send, recv, algo="oneshot", proto="simple")
            want = C.reduce_scatter(host, dt, "oneshot")
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"{op} {nbytes} B rank {r}")
        assert c.debug_state()["calls"] == before, "the call went through the ticket counter"
        assert c.check()[0] == "AR_OK"
    finally:
        c.close()


def test_empty_and_single_rank():
    for algo in ALGOS:
        for proto in PROTOS:
            run_allreduce(3, 0, "f32", algo, proto)
            run_allreduce(1, 1000, "bf16", algo, proto)
            run_allreduce(1, 1000, "i32", algo, proto, in_place=True)


# ------------------------------------------------------------ reduce-scatter
def run_rs(n, rc, dt, algo, proto, chunk=0, seed=0):
    host = inputs.rank_inputs(n, n * rc, dt, _dist(dt), seed=seed, cfg=200 + n)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(rc, dt) for _ in range(n)]
    _say("reduce_scatter", n, rc, dt, algo, proto, chunk)
    comm(n).reduce_scatter(send, recv, algo=algo, proto=proto, chunk_bytes=chunk)
    torch.cuda.synchronize()
    want = C.reduce_scatter(host, dt, algo, chunk_bytes=chunk or C.DEFAULT_CHUNK_BYTES)
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"reduce_scatter {algo}/{proto} {dt} N={n} rc={rc} rank {r}")
    assert comm(n).check()[0] == "AR_OK"


def run_ag(n, sc, dt, algo, proto, chunk=0, seed=0):
    host = inputs.rank_inputs(n, sc, dt, _dist(dt), seed=seed, cfg=300 + n)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(n * sc, dt) for _ in range(n)]
    _say("allgather", n, sc, dt, algo, proto, chunk)
    comm(n).allgather(send, recv, algo=algo, proto=proto, chunk_bytes=chunk)
    torch.cuda.synchronize()
    want = C.allgather(host, dt, algo, chunk_bytes=chunk or C.DEFAULT_CHUNK_BYTES)
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"allgather {algo}/{proto} {dt} N={n} sc={sc} rank {r}")
    assert comm(n).check()[0] == "AR_OK"


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("n", [2, 3, 8])
def test_reduce_scatter_matrix(n, algo, proto, dt):
    # odd counts leave every slice after the first misaligned (bf16: 2-byte)
    for rc in (1, 7, 1000, 17001):
        run_rs(n, rc, dt, algo, proto, seed=rc)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("n", [2, 3, 8])
def test_allgather_matrix(n, algo, proto, dt):
    for sc in (1, 7, 1000, 17001):
        run_ag(n, sc, dt, algo, proto, seed=sc)


@pytest.mark.parametrize("proto", PROTOS)
def test_rs_ag_ring_chunks(proto):
    for chunk in (16, 240, 4096):
        run_rs(4, 3001, "f32", "ring", proto, chunk=chunk)
        run_ag(4, 3001, "bf16", "ring", proto, chunk=chunk)


@pytest.mark.parametrize("proto", PROTOS)
def test_reduce_scatter_then_allgather_equals_allreduce(proto):
    n, rc = 8, 4096
    for dt in DTYPES:
        host = inputs.rank_inputs(n, n * rc, dt, _dist(dt), seed=3)
        send = [to_dev(x, dt) for x in host]
        for algo in ("twoshot", "ring"):
            shard = [empty(rc, dt) for _ in range(n)]
            full = [empty(n * rc, dt) for _ in range(n)]
            ar = [empty(n * rc, dt) for _ in range(n)]
            comm(n).reduce_scatter(send, shard, algo=algo, proto=proto)
            comm(n).allgather(shard, full, algo=algo, proto=proto)
            comm(n).allreduce(send, ar, algo=algo, proto=proto)
            torch.cuda.synchronize()
            for r in range(n):
                assert_same(to_host(full[r], dt), to_host(ar[r], dt), f"RS+AG vs AR {algo}/{proto} {dt}")


# ------------------------------------------------------ repeated calls, graphs
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
def test_back_to_back_calls_never_see_stale_flags(algo, proto):
    # The same buffers and staging, new data every call, no reset in between.
    n, count, dt = 8, 50000, "f32"
    send = [empty(count, dt) for _ in range(n)]
    recv = [empty(count, dt) for _ in range(n)]
    for it in range(6):
        host = inputs.rank_inputs(n, count, dt, "normal", seed=1000 + it)
        for t, x in zip(send, host):
            t.copy_(to_dev(x, dt))
        comm(n).allreduce(send, recv, algo=algo, proto=proto, chunk_bytes=64 << 10)
        torch.cuda.synchronize()
        want = C.allreduce(host, dt, algo, chunk_bytes=64 << 10)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"call {it} {algo}/{proto} rank {r}")


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
def test_hip_graph_replays(algo, proto):
    # Captured once; every replay must advance the device call counter, so a
    # replay never accepts the previous replay's flags.
    n, count, dt = 4, 20000, "bf16"
    send = [empty(count, dt) for _ in range(n)]
    recv = [empty(count, dt) for _ in range(n)]
    c = comm(n)
    stream = torch.cuda.Stream()
    c.allreduce(send, recv, algo=algo, proto=proto)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        c.allreduce(send, recv, algo=algo, proto=proto)
    torch.cuda.synchronize()
    for it in range(4):
        host = inputs.rank_inputs(n, count, dt, "normal", seed=2000 + it)
        for t, x in zip(send, host):
            t.copy_(to_dev(x, dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = C.allreduce(host, dt, algo)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"replay {it} {algo}/{proto} rank {r}")
        # eager work on the same communicator between replays
        c.allreduce(send, [empty(count, dt) for _ in range(n)], algo="ring", proto=proto)
        torch.cuda.synchronize()


# ------------------------------------------------------------- error paths
def test_argument_errors_are_reported():
    n = 4
    c = comm(n)
    good = [empty(64, "f32") for _ in range(n)]
    out = [empty(64, "f32") for _ in range(n)]
    with pytest.raises(ValueError):
        c.allreduce(good[:3], out[:3])
    with pytest.raises(ARError) as e:  # misaligned pointer
        c.allreduce([t[1:] for t in good], [t[1:] for t in out])
    assert e.value.status == 1
    with pytest.raises(ARError) as e:  # partial in place
        c.allreduce(good, [good[0]] + out[1:])
    assert e.value.status == 1
    with pytest.raises(ARError) as e:  # in-place reduce-scatter
        c.reduce_scatter(good, [t[:16] for t in good])
    assert e.value.status == 1
    with pytest.raises(ARError) as e:  # outputs overlap
        c.allreduce(good, [out[0]] * n)
    assert e.value.status == 1
    small = Comm(n, 1024, 0)
    with pytest.raises(ARError) as e:
        small.allreduce(good, out, proto="ll")  # no line staging provisioned
    assert e.value.status == 4
    big = [empty(1024, "f32") for _ in range(n)]
    with pytest.raises(ARError) as e:
        small.allreduce(big, [empty(1024, "f32") for _ in range(n)])
    assert e.value.status == 4
    small.close()
    assert c.check()[0] == "AR_OK"



def test_calls_that_never_wait_touch_no_counter():
    # One-shot (out of place), direct reduce-scatter and all-gather with
    # Simple never wait; when the grid covers every task they run without
    # the ticket counter and leave the call counter where it was.  Calls
    # that do wait still advance it by one.
    n, dt = 8, "bf16"
    c = Comm(n, 1 << 20, 0)
    host = inputs.rank_inputs(n, 4096, dt, "normal", seed=7)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(4096, dt) for _ in range(n)]
    _say("never-wait counters")
    before = c.debug_state()
    c.allreduce(send, recv, algo="oneshot")
    c.reduce_scatter(send, [empty(4096 // n, dt) for _ in range(n)], algo="oneshot")
    c.allgather([t[:512] for t in send], [empty(512 * n, dt) for _ in range(n)], algo="oneshot")
    mid = c.debug_state()
    assert (mid["calls"], mid["ticket"], mid["done"], mid["tasks_done"]) == \
        (before["calls"], 0, 0, before["tasks_done"])
    want = C.allreduce(host, dt, "oneshot")
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"oneshot rank {r}")
    c.allreduce(send, recv, algo="ring")
    after = c.debug_state()
    assert after["calls"] == before["calls"] + 1 and after["ticket"] == 0 and after["done"] == 0
    c.close()


def test_a_call_that_never_waits_completes_while_an_error_is_latched():
    # Forced from the host as in the timeout test below: the ring call times
    # out after 50 ms and latches the abort word.  A one-shot call that
    # follows before anyone checks cannot block, so it still runs in full;
    # the error stays latched for check().
    n = 4
    c = Comm(n, 1 << 20, 0)
    count = 64 * n
    host = inputs.rank_inputs(n, count, "f32", "normal", seed=5)
    send = [to_dev(x, "f32") for x in host]
    c.inject(1, 2, timeout_us=50_000)
    _say("latched abort, then oneshot")
    c.allreduce(send, [empty(count, "f32") for _ in range(n)], algo="ring")
    c.inject(-1, -1)
    recv = [empty(count, "f32") for _ in range(n)]
    c.allreduce(send, recv, algo="oneshot")
    torch.cuda.synchronize()
    want = C.allreduce(host, "f32", "oneshot")
    for r in range(n):
        assert_same(to_host(recv[r], "f32"), want[r], f"oneshot after abort, rank {r}")
    assert c.check()[0] == "AR_ERR_TIMEOUT"
    c.reset()
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("algo,n,rank,step", [("ring", 4, 1, 2), ("ring", 8, 5, 9), ("twoshot", 4, 2, 0)])
def test_withheld_signal_times_out_and_names_the_blocked_rank(algo, n, rank, step):
    # Forced from the host: one rank program skips one signal and waits are
    # limited to 50 ms, so every wave of the kernel still exits.
    from oracle import sim

    c = Comm(n, 1 << 20, 0)
    count = 64 * n  # one tile per block: nothing else is still running at the timeout
    host = inputs.rank_inputs(n, count, "f32", "normal", seed=4)
    send = [to_dev(x, "f32") for x in host]
    recv = [empty(count, "f32") for _ in range(n)]
    c.inject(rank, step, timeout_us=50_000)
    _say("inject", algo, n, rank, step)
    c.allreduce(send, recv, algo=algo)
    status, r, s = c.check()
    assert status == "AR_ERR_TIMEOUT"
    _, first = sim.blocked("allreduce", algo, n, withheld=(rank, step))
    assert (r, s) == first
    with pytest.raises(ARError) as e:
        c.allreduce(send, recv, algo=algo)
    assert e.value.status == 7
    c.inject(-1, -1)
    c.reset()
    run_ok = [empty(count, "f32") for _ in range(n)]
    c.allreduce(send, run_ok, algo=algo)
    torch.cuda.synchronize()
    want = C.allreduce(host, "f32", algo)
    assert_same(to_host(run_ok[0], "f32"), want[0], "after reset")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("algo,proto,n,rank,step", [
    ("oneshot", "ll", 4, 2, 0), ("oneshot", "ll128", 8, 0, 0),
    ("twoshot", "ll", 4, 1, 0), ("twoshot", "ll128", 8, 3, 1),
    ("ring", "ll", 4, 1, 2), ("ring", "ll128", 8, 5, 9), ("ring", "ll128", 3, 0, 0)])
def test_withheld_line_flags_time_out_and_name_the_blocked_rank(algo, proto, n, rank, step):
    # Forced from the host: one rank program writes its lines of one step
    # without their flags (LL: does not write them) and waits are limited to
    # 50 ms; every wave of the kernel still exits.  The blocked (rank, step)
    # reported is the first one the oracle's transfer graph predicts.
    from oracle import sim

    c = Comm(n, 1 << 20, 1 << 20)
    count = 64 * n  # one tile per block: nothing else is still running at the timeout
    host = inputs.rank_inputs(n, count, "f32", "normal", seed=5)
    send = [to_dev(x, "f32") for x in host]
    recv = [empty(count, "f32") for _ in range(n)]
    c.inject(rank, step, timeout_us=50_000)
    _say("inject-lines", algo, proto, n, rank, step)
    c.allreduce(send, recv, algo=algo, proto=proto)
    status, r, s = c.check()
    assert status == "AR_ERR_TIMEOUT"
    _, first = sim.blocked("allreduce", algo, n, withheld=(rank, step), proto=proto)
    assert (r, s) == first
    with pytest.raises(ARError) as e:
        c.allreduce(send, recv, algo=algo, proto=proto)
    assert e.value.status == 7
    c.inject(-1, -1)
    c.reset()
    run_ok = [empty(count, "f32") for _ in range(n)]
    c.allreduce(send, run_ok, algo=algo, proto=proto)
    torch.cuda.synchronize()
    want = C.allreduce(host, "f32", algo)
    for q in range(n):
        assert_same(to_host(run_ok[q], "f32"), want[q], f"after reset rank {q}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("op,proto", [("reduce_scatter", "ll128"), ("allgather", "ll")])
def test_withheld_line_flags_direct_rs_ag(op, proto):
    from oracle import sim

    n, rank = 4, 2
    c = Comm(n, 1 << 20, 1 << 20)
    shard = 64
    full = inputs.rank_inputs(n, n * shard, "f32", "normal", seed=6)
    if op == "reduce_scatter":
        send = [to_dev(x, "f32") for x in full]
        recv = [empty(shard, "f32") for _ in range(n)]
    else:
        send = [to_dev(x[:shard], "f32") for x in full]
        recv = [empty(n * shard, "f32") for _ in range(n)]
    c.inject(rank, 0, timeout_us=50_000)
    _say("inject-lines", op, proto, n, rank)
    getattr(c, op)(send, recv, algo="oneshot", proto=proto)
    status, r, s = c.check()
    assert status == "AR_ERR_TIMEOUT"
    assert (r, s) == sim.blocked(op, "twoshot", n, withheld=(rank, 0), proto=proto)[1]
    c.inject(-1, -1)
    c.reset()
    getattr(c, op)(send, recv, algo="oneshot", proto=proto)
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("proto", ["ll", "ll128"])
@pytest.mark.parametrize("n", [2, 5, 8])
@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
def test_small_line_one_shot_runs_one_workgroup_per_tile_and_rank(dt, n, proto):
    # Decode-sized one-shot calls over LL / LL128 run each (tile, rank) as one
    # workgroup with no ticket counter; the call log shows it, and the results
    # equal the oracle's out of place and in place.  With a workgroup budget
    # below the grid the same call takes the ticketed schedule.  LL's largest
    # case (80 KiB per rank in 4-byte types: 20 tiles) needs up to 160
    # workgroups, past LL128's cap of 64.
    c = Comm(n, 1 << 20, 1 << 20)
    for count in (1, 999, 5120, 40960 if proto == "ll128" else 3000, 20480):
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=count, cfg=80)
        want = C.allreduce(host, dt, "oneshot")
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        _say("coloc", dt, n, proto, count)
        c.allreduce(send, recv, algo="oneshot", proto=proto)
        torch.cuda.synchronize()
        assert c.debug_calls(1)[0]["counter_free"] == 1, (dt, n, proto, count)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"coloc {proto} {dt} N={n} count={count} rank {r}")
        c.allreduce(send, None, algo="oneshot", proto=proto)  # in place
        torch.cuda.synchronize()
        for r in range(n):
            assert_same(to_host(send[r], dt), want[r], f"coloc in place {proto} {dt} N={n} count={count} rank {r}")
    # A budget below the grid (20480 elements: at least 3 tiles per rank for
    # either protocol, so more than max(budget, N) workgroups).
    c.set_max_workgroups(n - 1 if n > 2 else 1)
    host = inputs.rank_inputs(n, 20480, dt, _dist(dt), seed=1, cfg=81)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(20480, dt) for _ in range(n)]
    c.allreduce(send, recv, algo="oneshot", proto=proto)
    torch.cuda.synchronize()
    assert c.debug_calls(1)[0]["counter_free"] == 0
    want = C.allreduce(host, dt, "oneshot")
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"budget {proto} {dt} N={n} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


def test_call_log_after_three_calls():
    n = 4
    c = Comm(n, 1 << 20, 1 << 20)
    host = inputs.rank_inputs(n, 4096, "f32", "normal", seed=7)
    send = [to_dev(x, "f32") for x in host]
    recv = [empty(4096, "f32") for _ in range(n)]
    c.allreduce(send, recv, algo="ring", proto="simple")
    c.reduce_scatter(send, [t[:1024] for t in recv], algo="oneshot", proto="ll128")
    c.allreduce(send, recv, algo="auto", proto="auto")
    torch.cuda.synchronize()
    recs = c.debug_calls()
    assert [r["seq"] for r in recs] == [1, 2, 3]
    assert [(r["op"], r["algo"], r["proto"]) for r in recs[:2]] == [
        ("allreduce", "ring", "simple"), ("reduce_scatter", "oneshot", "ll128")]
    assert recs[2]["algo"] != "auto" and recs[2]["proto"] in ("simple", "ll", "ll128")
    assert [r["count"] for r in recs] == [4096, 1024, 4096]
    assert all(r["nranks"] == n and r["grid"] >= 1 and r["ntasks"] >= 1 for r in recs)
    assert [r["seq"] for r in c.debug_calls(2)] == [2, 3]
    assert c.check()[0] == "AR_OK"
    c.close()


def test_ar_debug_prints_each_plan_and_the_log_on_a_timeout():
    import os
    import subprocess
    code = (
        "import torch\n"
        "from all_reduce_reduction_rank_amd import Comm\n"
        "c = Comm(4, 1 << 20, 0)\n"
        "x = [torch.ones(256, device='cuda') for _ in range(4)]\n"
        "y = [torch.empty(256, device='cuda') for _ in range(4)]\n"
        "c.allreduce(x, y, algo='twoshot')\n"
        "c.inject(1, 2, timeout_us=50000)\n"
        "c.allreduce(x, y, algo='ring')\n"
        "print(c.check())\n")
    env = dict(os.environ, AR_DEBUG="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stderr
    err = res.stderr
    assert "[ar] call 1: allreduce twoshot/simple f32 N=4 count=256" in err
    assert "[ar] call 2: allreduce ring/simple f32 N=4 count=256" in err
    assert "[ar] latched error 6: first blocked wait rank 2 step 3" in err
    assert "[ar]   call 1: allreduce twoshot" in err and "[ar]   call 2: allreduce ring" in err
    assert "AR_ERR_TIMEOUT" in res.stdout


# ------------------------------------------------------ automatic choice
@pytest.mark.parametrize("n", [2, 3, 8])
@pytest.mark.parametrize("dt", ["f32", "bf16", "i32"])
def test_auto_choice_matches_the_oracle_of_the_chosen_schedule(n, dt):
    from all_reduce_reduction_rank_amd import select

    c = comm(n)
    for count in (3, 4096, 70001, 1 << 18):
        host = inputs.rank_inputs(n, count, dt, _dist(dt), seed=count, cfg=40)
        send = [to_dev(x, dt) for x in host]
        recv = [empty(count, dt) for _ in range(n)]
        algo, proto, _ = select(n, "allreduce", count, dt, max_line_bytes_per_rank=LINE_BYTES)
        print("CASE auto", n, dt, count, algo, proto, flush=True, file=sys.stderr)
        c.allreduce(send, recv, algo="auto", proto="auto")
        torch.cuda.synchronize()
        want = C.allreduce(host, dt, algo)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"auto ({algo}/{proto}) N={n} {dt} count={count} rank {r}")
    assert c.check()[0] == "AR_OK"


@pytest.mark.parametrize("op", ["reduce_scatter", "allgather"])
def test_auto_choice_for_reduce_scatter_and_all_gather(op):
    from all_reduce_reduction_rank_amd import select

    n, dt, cnt = 4, "f32", 5000
    c = comm(n)
    total = n * cnt
    host = inputs.rank_inputs(n, total if op == "reduce_scatter" else cnt, dt, "normal", seed=5, cfg=41)
    send = [to_dev(x, dt) for x in host]
    recv = [empty(cnt if op == "reduce_scatter" else total, dt) for _ in range(n)]
    algo, proto, _ = select(n, op, cnt, dt, max_line_bytes_per_rank=LINE_BYTES)
    getattr(c, op)(send, recv, algo="auto", proto="auto")
    torch.cuda.synchronize()
    want = getattr(C, op)(host, dt, algo)
    for r in range(n):
        assert_same(to_host(recv[r], dt), want[r], f"auto {op} ({algo}/{proto}) rank {r}")


# ------------------------------------------------------ workgroup budget
@pytest.mark.parametrize("budget", [1, 2, 5, 64])
def test_workgroup_budget_keeps_results(budget):
    n, dt, count = 4, "f32", 300001
    c = Comm(n, count * 4, count * 4)
    c.set_max_workgroups(budget)
    host = inputs.rank_inputs(n, count, dt, "normal", seed=budget, cfg=42)
    send = [to_dev(x, dt) for x in host]
    for algo in ("oneshot", "twoshot", "ring"):
        want = C.allreduce(host, dt, algo)
        for proto in ("simple", "ll", "ll128"):
            print("CASE budget", budget, algo, proto, flush=True, file=sys.stderr)
            recv = [empty(count, dt) for _ in range(n)]
            c.allreduce(send, recv, algo=algo, proto=proto)
            torch.cuda.synchronize()
            for r in range(n):
                assert_same(to_host(recv[r], dt), want[r], f"budget {budget} {algo}/{proto} rank {r}")
    # in place one-shot: the read-done barrier still gets N workgroups
    print("CASE budget in-place", budget, flush=True, file=sys.stderr)
    inplace = [to_dev(x, dt) for x in host]
    c.allreduce(inplace, None, algo="oneshot")
    torch.cuda.synchronize()
    want = C.allreduce(host, dt, "oneshot")
    for r in range(n):
        assert_same(to_host(inplace[r], dt), want[r], f"budget {budget} in-place rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


# ------------------------------------------------------ double binary tree
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("n", [2, 3, 4, 5, 7, 8])
def test_tree_allreduce(n, dt):
    # 1 element (half 1 empty), ragged halves, several 32 KiB tiles per half.
    for count in (1, 7, 1000, 70001, 300003):
        run_allreduce(n, count, dt, "tree", "simple", seed=count)


def test_tree_in_place_ones_and_single_rank():
    for dt in DTYPES:
        for n, count in ((2, 4096), (5, 33333), (8, 100001)):
            run_allreduce(n, count, dt, "tree", "simple", seed=3, in_place=True)
        run_allreduce(8, 128, dt, "tree", "simple", dist="ones")
    run_allreduce(1, 999, "f32", "tree", "simple")


def test_tree_graph_replays():
    n, count, dt = 6, 50001, "f32"
    c = comm(n)
    send = [empty(count, dt) for _ in range(n)]
    recv = [empty(count, dt) for _ in range(n)]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        c.allreduce(send, recv, algo="tree", proto="simple")
    torch.cuda.synchronize()
    for it in range(3):
        host = inputs.rank_inputs(n, count, dt, "normal", seed=3000 + it)
        for t, x in zip(send, host):
            t.copy_(to_dev(x, dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = C.allreduce(host, dt, "tree")
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"tree replay {it} rank {r}")
        c.allreduce(send, [empty(count, dt) for _ in range(n)], algo="ring")  # eager work between replays
        torch.cuda.synchronize()


def test_tree_with_line_protocols_or_rs_ag_is_unsupported():
    n = 4
    c = comm(n)
    x = [empty(64, "f32") for _ in range(n)]
    y = [empty(64, "f32") for _ in range(n)]
    for proto in ("ll", "ll128"):
        with pytest.raises(ARError) as e:
            c.allreduce(x, y, algo="tree", proto=proto)
        assert e.value.status == 2
    with pytest.raises(ARError):
        c.reduce_scatter(x, [empty(16, "f32") for _ in range(n)], algo="tree")
    assert c.check()[0] == "AR_OK"
