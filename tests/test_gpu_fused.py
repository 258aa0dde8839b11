"""GPU parity of the fused all-reduce + RMSNorm epilogue (ar_allreduce_rmsnorm).

The updated residual (and, with a zero residual, the all-reduce sum itself)
must match the oracle bit for bit.  The normalized output is computed in
fp32 on the GPU and in fp64 by the oracle; the tolerance follows from the
GPU's arithmetic: the sum of squares of a row is a chain of at most ~60
fp32 additions of non-negative terms (relative error <= 60 * 2^-24 =
3.6e-6), the square root halves it, and the division, square root and two
products add four roundings: under 2.2e-6 relative, so fp32 outputs must
agree within 4e-6 relative and bf16 outputs (whose rounding step is 2^-9)
within one bf16 unit in the last place.
"""

import sys

import numpy as np
import pytest
import torch

from all_reduce_reduction_rank_amd import ARError, Comm, inputs
from oracle import bf16, fused
from tests.gpu_util import assert_same, empty, to_dev, to_host

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def _say(*what):
    print("CASE", *what, flush=True, file=sys.stderr)


def _close(got, want, dt, what):
    if dt == "bf16":
        d = bf16.ulp_distance(got, want)
        assert d.max() <= 1, f"{what}: {int((d > 1).sum())} elements beyond 1 ulp, max {d.max()}"
    else:
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        bound = 4e-6 * np.abs(want.astype(np.float64)) + 1e-30
        bad = np.flatnonzero(err > bound)
        assert bad.size == 0, f"{what}: {bad.size} elements off, first {bad[:3]}: {got[bad[:3]]} vs {want[bad[:3]]}"


def run_fused(n, rows, hidden, dt, with_residual, eps=1e-6, seed=0, comm=None, zero_residual=False):
    _say("fused", n, rows, hidden, dt, "residual" if with_residual else "", "zero" if zero_residual else "")
    count = rows * hidden
    x = inputs.rank_inputs(n, count, dt, "normal", seed=seed, cfg=70)
    w = inputs.rank_inputs(1, hidden, dt, "normal", seed=seed + 1, cfg=71)[0]
    res = None
    if with_residual:
        res = inputs.rank_inputs(n, count, dt, "normal", seed=seed + 2, cfg=72)
        if zero_residual:
            res = [np.zeros_like(v) for v in res]
    c = comm or Comm(n, count * (2 if dt == "bf16" else 4), 0)
    send = [to_dev(v, dt).view(rows, hidden) for v in x]
    out = [empty(count, dt).view(rows, hidden) for _ in range(n)]
    res_dev = [to_dev(v, dt).view(rows, hidden) for v in res] if res is not None else None
    c.allreduce_rmsnorm(send, out, to_dev(w, dt), eps=eps, residual=res_dev)
    torch.cuda.synchronize()
    want_out, want_res = fused.allreduce_rmsnorm(x, res, w, rows, hidden, eps, dt)
    for r in range(n):
        _close(to_host(out[r].view(-1), dt), want_out[r], dt, f"out N={n} {rows}x{hidden} {dt} rank {r}")
        if res is not None:
            assert_same(to_host(res_dev[r].view(-1), dt), want_res[r], f"residual N={n} {dt} rank {r}")
    if comm is None:
        c.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [3, 8])
def test_fused_prefill_rows_placed_by_die(n, dt):
    # More (row, rank) items than the grid and N inputs beyond one die's
    # L2: each row's N items run on one die, the grid cut to whole 8 N
    # blocks of workgroups.  The TP prefill shape [512, 5120] and a
    # ragged row count.
    for rows, hidden in ((512, 5120), (301, 2048)):
        run_fused(n, rows, hidden, dt, with_residual=True, seed=rows + n)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_fused_matches_oracle(n, dt):
    # (160, 1024): at N=8, 1280 (row, rank) items, more than one per
    # workgroup of the grid -- the kernel then loads the weights after the sum
    for rows, hidden in ((1, 5120), (7, 640), (64, 5120), (3, 12288), (5, 8), (160, 1024)):
        if hidden * (2 if dt == "bf16" else 4) % 16:
            continue
        run_fused(n, rows, hidden, dt, with_residual=False, seed=rows)
        run_fused(n, rows, hidden, dt, with_residual=True, seed=rows + 10)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_zero_residual_returns_the_all_reduce_sum_bit_exactly(dt):
    # h = a + 0 = a: the updated residual is the one-shot all-reduce result
    run_fused(8, 16, 5120, dt, with_residual=True, zero_residual=True, seed=3)


def test_tp_decode_and_prefill_shapes():
    # TP activations: [tokens, 5120] bf16 at N=8, tokens 1 and 512
    c = Comm(8, 512 * 5120 * 2, 0)
    for tokens in (1, 512):
        run_fused(8, tokens, 5120, "bf16", with_residual=True, eps=1e-5, seed=tokens, comm=c)
    c.close()


def test_graph_replays_of_the_fused_call():
    n, rows, hidden, dt = 4, 32, 2048, "bf16"
    c = Comm(n, rows * hidden * 2, 0)
    send = [empty(rows * hidden, dt).view(rows, hidden) for _ in range(n)]
    out = [empty(rows * hidden, dt).view(rows, hidden) for _ in range(n)]
    w_host = inputs.rank_inputs(1, hidden, dt, "normal", seed=8, cfg=71)[0]
    w = to_dev(w_host, dt)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        c.allreduce_rmsnorm(send, out, w, eps=1e-6)
    torch.cuda.synchronize()
    for it in range(3):
        x = inputs.rank_inputs(n, rows * hidden, dt, "normal", seed=40 + it, cfg=70)
        for t, v in zip(send, x):
            t.view(-1).copy_(to_dev(v, dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want, _ = fused.allreduce_rmsnorm(x, None, w_host, rows, hidden, 1e-6, dt)
        for r in range(n):
            _close(to_host(out[r].view(-1), dt), want[r], dt, f"replay {it} rank {r}")
    c.close()


def test_fused_argument_errors():
    n, rows, hidden = 2, 4, 64
    c = Comm(n, 1 << 20, 0)
    mk = lambda dt, h=hidden: [torch.zeros(rows, h, dtype=dt, device="cuda") for _ in range(n)]  # noqa: E731
    w = torch.ones(hidden, dtype=torch.float32, device="cuda")
    with pytest.raises(ARError) as e:  # integers: not normalizable
        c.allreduce_rmsnorm(mk(torch.int32), mk(torch.int32), torch.ones(hidden, dtype=torch.int32, device="cuda"))
    assert e.value.status == 2
    with pytest.raises(ARError) as e:  # rows of partial 16-byte vectors
        c.allreduce_rmsnorm(mk(torch.float32, 6), mk(torch.float32, 6), torch.ones(6, device="cuda"))
    assert e.value.status == 1
    with pytest.raises(ARError) as e:  # hidden beyond the LDS row buffer
        c.allreduce_rmsnorm(mk(torch.float32, 16384), mk(torch.float32, 16384), torch.ones(16384, device="cuda"))
    assert e.value.status == 2
    s = mk(torch.float32)
    with pytest.raises(ARError) as e:  # in place is not allowed
        c.allreduce_rmsnorm(s, s, w)
    assert e.value.status == 1
    assert c.check()[0] == "AR_OK"
    c.close()
