"""GPU: no kernel writes outside its output.  Every rank's output is a view
into one allocation with guard bytes before, between and after the ranks'
outputs; after each call the guards must hold their pattern and the outputs
must equal the oracle's.  Sizes are chosen so that blocks and tiles end in
the middle of an LL128 line (and of a 16-byte vector), where padding lanes
carry no payload."""

import sys

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import Comm, inputs
from oracle import collectives as C
from tests.gpu_util import TORCH, assert_same, to_dev, to_host

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes before, between and after the ranks' outputs
ESIZE = {"f32": 4, "bf16": 2, "i32": 4}
_COMMS = {}


def _comm(n):
    if n not in _COMMS:
        _COMMS[n] = Comm(n, 8 << 20, 8 << 20)
    return _COMMS[n]


def _guarded_outputs(n, count, dt):
    """One uint8 arena: [guard | out 0 | guard | out 1 | ... | guard]."""
    nb = count * ESIZE[dt]
    stride = GUARD + (nb + 255) // 256 * 256
    arena = torch.empty(GUARD + n * stride, dtype=torch.uint8, device="cuda")
    arena.fill_(0x5C)
    outs = [arena[GUARD + r * stride:GUARD + r * stride + nb].view(TORCH[dt]) for r in range(n)]
    keep = torch.ones(arena.numel(), dtype=torch.bool)
    for r in range(n):
        keep[GUARD + r * stride:GUARD + r * stride + nb] = False
    return arena, outs, keep


def _check_guards(arena, keep, what):
    host = arena.cpu().numpy()
    bad = np.flatnonzero((host != 0x5C) & keep.numpy())
    assert bad.size == 0, f"{what}: {bad.size} guard bytes written, first at arena offsets {bad[:8]}"


CASES = [(algo, proto) for algo in ("oneshot", "twoshot", "ring") for proto in ("simple", "ll", "ll128")] + \
        [("tree", "simple")]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n", [3, 8])
def test_allreduce_writes_only_its_outputs(n, dt):
    # bf16 5120: 1280-byte blocks at N=8 (10 2/3 LL128 lines); f32 3001: ragged blocks and tail
    for count in ((5120, 40960 + 37) if dt == "bf16" else (3001, 20000 + 3)):
        host = inputs.rank_inputs(n, count, dt, "normal", seed=count, cfg=80)
        send = [to_dev(x, dt) for x in host]
        for algo, proto in CASES:
            print("CASE bounds allreduce", n, dt, count, algo, proto, file=sys.stderr, flush=True)
            arena, recv, keep = _guarded_outputs(n, count, dt)
            _comm(n).allreduce(send, recv, algo=algo, proto=proto)
            torch.cuda.synchronize()
            _check_guards(arena, keep, f"allreduce {algo}/{proto} N={n} {dt} count={count}")
            want = C.allreduce(host, dt, algo)
            for r in range(n):
                assert_same(to_host(recv[r], dt), want[r], f"allreduce {algo}/{proto} rank {r}")


@pytest.mark.parametrize("op", ["reduce_scatter", "allgather"])
@pytest.mark.parametrize("n", [3, 8])
def test_rs_ag_write_only_their_outputs(op, n):
    dt = "bf16"
    for shard in (1283, 7):
        full = n * shard
        if op == "reduce_scatter":
            host = inputs.rank_inputs(n, full, dt, "normal", seed=shard, cfg=81)
            out_count = shard
        else:
            host = inputs.rank_inputs(n, shard, dt, "normal", seed=shard, cfg=82)
            out_count = full
        send = [to_dev(x, dt) for x in host]
        for algo in ("oneshot", "ring"):
            for proto in ("simple", "ll", "ll128"):
                print("CASE bounds", op, n, shard, algo, proto, file=sys.stderr, flush=True)
                arena, recv, keep = _guarded_outputs(n, out_count, dt)
                getattr(_comm(n), op)(send, recv, algo=algo, proto=proto)
                torch.cuda.synchronize()
                _check_guards(arena, keep, f"{op} {algo}/{proto} N={n} shard={shard}")
                want = C.reduce_scatter(host, dt, algo) if op == "reduce_scatter" else C.allgather(host, dt, algo)
                for r in range(n):
                    assert_same(to_host(recv[r], dt), want[r], f"{op} {algo}/{proto} rank {r}")
