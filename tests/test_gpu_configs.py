"""GPU parity at the workloads' full sizes.

Full-size buffers are drawn on the GPU (seeded torch generator).  Outputs are
checked at sampled positions: the oracle runs on a reduced problem made of
the sampled positions of every block, which keeps each element's block --
and so its summation order (one-shot / two-shot: ranks in ascending order;
ring: starting after the block's owner) -- so the oracle's result at those
positions is exactly what the full-size call must produce there.  Smaller
sizes are compared in full.
"""

import sys

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import Comm, inputs
from oracle import collectives as C, geometry
from tests.gpu_util import assert_same, to_dev, to_host

pytestmark = pytest.mark.gpu

ALGOS = ("oneshot", "twoshot", "ring")
PROTOS = ("simple", "ll", "ll128")
ESIZE = {"f32": 4, "bf16": 2, "i32": 4}


def _say(*what):
    print("CASE", *what, flush=True, file=sys.stderr)


def _samples(lo, hi, m, rng):
    """m sorted positions in [lo, hi) including both ends (fewer if short)."""
    if hi - lo <= m:
        return np.arange(lo, hi)
    mid = rng.choice(np.arange(lo + 1, hi - 1), size=m - 2, replace=False)
    return np.sort(np.concatenate([[lo, hi - 1], mid]))


def _gather(tensors, idx, dt):
    t_idx = torch.from_numpy(idx).cuda()
    return [to_host(t.index_select(0, t_idx), dt) for t in tensors]


def check_allreduce_sampled(n, count, dt, algo, proto, dist, chunk=0, m=2048, seed=0):
    _say("allreduce-full", n, count, dt, algo, proto, dist, chunk)
    send = inputs.device_rank_inputs(n, count, dt, dist, seed=seed, cfg=50)
    recv = [torch.empty_like(t) for t in send]
    es = ESIZE[dt]
    line = count * es if proto != "simple" else 0
    c = Comm(n, count * es, line)
    c.allreduce(send, recv, algo=algo, proto=proto, chunk_bytes=chunk)
    torch.cuda.synchronize()
    assert c.check()[0] == "AR_OK"
    c.close()
    rng = np.random.default_rng(seed)
    a = geometry.vec_elems(dt)
    per = (m // a) * a
    blocks = geometry.ar_blocks(count, n, dt)
    idx_parts = []
    for lo, hi in blocks:
        pos = _samples(lo, hi, per, rng) if hi > lo else np.arange(0)
        assert len(pos) in (0, per) or hi - lo < per
        idx_parts.append(pos)
    if any(0 < len(p) < per for p in idx_parts) or any(len(p) == 0 for p in idx_parts):
        pytest.skip("blocks too short for the reduced problem; small sizes are compared in full")
    idx = np.concatenate(idx_parts)
    red_in = _gather(send, idx, dt)
    want = C.allreduce(red_in, dt, algo, chunk_bytes=chunk or C.DEFAULT_CHUNK_BYTES)
    got = _gather(recv, idx, dt)
    for r in range(n):
        assert_same(got[r], want[r], f"allreduce {algo}/{proto} {dt} N={n} count={count} rank {r}")
    del send, recv
    torch.cuda.empty_cache()


# ------------------------------------------------- gradient buckets (N=8 fp32)
@pytest.mark.parametrize("mib", [25, 256])
def test_gradient_bucket_ring_512k_chunks(mib):
    count = mib * (1 << 20) // 4
    check_allreduce_sampled(8, count, "f32", "ring", "simple", "normal_1e-3", chunk=512 << 10)


@pytest.mark.parametrize("algo", ["oneshot", "twoshot"])
def test_gradient_bucket_256mib_other_algorithms(algo):
    check_allreduce_sampled(8, 64 << 20, "f32", algo, "simple", "normal_1e-3")


# ------------------------------------------ TP activations (N=8 bf16, full)
@pytest.mark.parametrize("tokens", [1, 8, 64, 512])
def test_tp_activations_bf16_full_compare(tokens):
    n, count = 8, tokens * 5120
    host = inputs.rank_inputs(n, count, "bf16", "normal", seed=tokens, cfg=2)
    send = [to_dev(x, "bf16") for x in host]
    c = Comm(n, count * 2, count * 2)
    for algo in ("oneshot", "twoshot"):
        want = C.allreduce(host, "bf16", algo)
        for proto in PROTOS:
            _say("tp", tokens, algo, proto)
            recv = [torch.empty_like(t) for t in send]
            c.allreduce(send, recv, algo=algo, proto=proto)
            torch.cuda.synchronize()
            for r in range(n):
                assert_same(to_host(recv[r], "bf16"), want[r], f"tp{tokens} {algo}/{proto} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


# ----------------------------------------------- integer path (int32, N=4,8)
@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("mib", [1, 4, 16, 64])
def test_int32_ring_allreduce_rs_ag(n, mib):
    es, m = 4, 1024
    total = mib * (1 << 20) // es  # elements of the full per-rank buffer
    check_allreduce_sampled(n, total, "i32", "ring", "simple", "int20", chunk=512 << 10, m=m, seed=mib)
    rng = np.random.default_rng(mib)
    rc = total // n
    c = Comm(n, total * es, 0)
    # reduce-scatter: send N*rc per rank, receive rc
    send = inputs.device_rank_inputs(n, n * rc, "i32", "int20", seed=mib, cfg=3)
    recv = [torch.empty(rc, dtype=torch.int32, device="cuda") for _ in range(n)]
    for algo in ("ring", "twoshot"):
        _say("rs-full", n, mib, algo)
        c.reduce_scatter(send, recv, algo=algo, chunk_bytes=512 << 10)
        torch.cuda.synchronize()
        pos = _samples(0, rc, m, rng)
        red_in = _gather(send, np.concatenate([j * rc + pos for j in range(n)]), "i32")
        want = C.reduce_scatter(red_in, "i32", algo)
        got = _gather(recv, pos, "i32")
        for r in range(n):
            assert_same(got[r], want[r], f"reduce_scatter {algo} N={n} {mib} MiB rank {r}")
    # all-gather: send sc per rank, receive N*sc
    sc = rc
    send_ag = [t[:sc] for t in send]
    recv_ag = [torch.empty(n * sc, dtype=torch.int32, device="cuda") for _ in range(n)]
    for algo in ("ring", "twoshot"):
        _say("ag-full", n, mib, algo)
        c.allgather(send_ag, recv_ag, algo=algo, chunk_bytes=512 << 10)
        torch.cuda.synchronize()
        pos = _samples(0, sc, m, rng)
        red_in = _gather(send_ag, pos, "i32")
        want = C.allgather(red_in, "i32", algo)
        got = _gather(recv_ag, np.concatenate([j * sc + pos for j in range(n)]), "i32")
        for r in range(n):
            assert_same(got[r], want[r], f"allgather {algo} N={n} {mib} MiB rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


# --------------------------------------------------- message-size sweep
SWEEP_SMALL = [8 * 4 ** k for k in range(9)]  # 8 B .. 512 KiB: full compare


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_sweep_small_sizes_full_compare(n, dt):
    es = ESIZE[dt]
    c = Comm(n, SWEEP_SMALL[-1], SWEEP_SMALL[-1])
    for nbytes in SWEEP_SMALL:
        count = nbytes // es
        host = inputs.rank_inputs(n, count, dt, "normal", seed=nbytes, cfg=5)
        send = [to_dev(x, dt) for x in host]
        for algo in ALGOS:
            want = C.allreduce(host, dt, algo)
            for proto in PROTOS:
                recv = [torch.empty_like(t) for t in send]
                c.allreduce(send, recv, algo=algo, proto=proto)
                torch.cuda.synchronize()
                for r in range(n):
                    assert_same(to_host(recv[r], dt), want[r], f"sweep {nbytes} B {algo}/{proto} {dt} N={n}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("mib", [8, 128])
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
def test_sweep_large_sizes_sampled(algo, proto, mib):
    check_allreduce_sampled(8, mib * (1 << 20) // 4, "f32", algo, proto, "normal", seed=mib)


@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_256mib_sampled(algo):
    # the bf16 bandwidth workload at full size, as the bench launches it
    check_allreduce_sampled(8, (256 << 20) // 2, "bf16", algo, "simple", "normal", chunk=512 << 10, seed=16)


@pytest.mark.parametrize("algo", ALGOS)
def test_sweep_one_gib(algo):
    check_allreduce_sampled(8, (1 << 30) // 4, "f32", algo, "simple", "normal", seed=30)


def test_sweep_one_gib_ll128_ring():
    check_allreduce_sampled(8, (1 << 30) // 4, "f32", "ring", "ll128", "normal", seed=31)


# ------------------------------------------------------------- stress
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("algo", ALGOS)
def test_repeated_calls_at_8mib_stay_exact(algo, proto):
    # Many back-to-back calls with fresh data: a producer/consumer ordering
    # hole would show up as a stale value somewhere.
    n, count, dt = 8, 2 << 20, "f32"
    c = Comm(n, count * 4, count * 4)
    recv = [torch.empty(count, dtype=torch.float32, device="cuda") for _ in range(n)]
    for it in range(3):
        send = inputs.device_rank_inputs(n, count, dt, "normal", seed=100 + it, cfg=7)
        c.allreduce(send, recv, algo=algo, proto=proto, chunk_bytes=256 << 10)
        torch.cuda.synchronize()
        want = C.allreduce([to_host(t, dt) for t in send], dt, algo, chunk_bytes=256 << 10)
        for r in range(n):
            assert_same(to_host(recv[r], dt), want[r], f"stress {algo}/{proto} call {it} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


@pytest.mark.parametrize("algo", ALGOS)
def test_in_place_at_8mib(algo):
    n, count, dt = 8, 2 << 20, "f32"
    c = Comm(n, count * 4, 0)
    send = inputs.device_rank_inputs(n, count, dt, "normal", seed=7, cfg=8)
    want = C.allreduce([to_host(t, dt) for t in send], dt, algo)
    c.allreduce(send, None, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert_same(to_host(send[r], dt), want[r], f"in place {algo} rank {r}")
    assert c.check()[0] == "AR_OK"
    c.close()


# ------------------------------------------- tree at the gradient-bucket size
def test_tree_gradient_bucket_256mib_sampled():
    # The tree's order depends only on the half an element is in, so a
    # reduced problem made of `per` samples of each half (in order) keeps it.
    n, count, dt = 8, 64 << 20, "f32"
    _say("tree-full", n, count)
    send = inputs.device_rank_inputs(n, count, dt, "normal_1e-3", seed=1, cfg=51)
    recv = [torch.empty_like(t) for t in send]
    c = Comm(n, count * 4, 0)
    c.allreduce(send, recv, algo="tree", proto="simple")
    torch.cuda.synchronize()
    assert c.check()[0] == "AR_OK"
    c.close()
    rng = np.random.default_rng(1)
    per = 2048
    halves = geometry.ar_blocks(count, 2, dt)
    idx = np.concatenate([_samples(lo, hi, per, rng) for lo, hi in halves])
    red_in = _gather(send, idx, dt)
    assert geometry.ar_blocks(len(idx), 2, dt) == [(0, per), (per, 2 * per)]
    want = C.allreduce(red_in, dt, "tree")
    got = _gather(recv, idx, dt)
    for r in range(n):
        assert_same(got[r], want[r], f"tree 256 MiB rank {r}")
    del send, recv
    torch.cuda.empty_cache()
