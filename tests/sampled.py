"""Parity of full-size GPU calls at sampled positions (GPU test helper).

A full-size buffer is too large for the oracle, so the oracle runs on a
reduced problem made of the sampled positions of every block.  Each sampled
element keeps its block, and so its summation order (one-shot and two-shot:
ranks in ascending order; ring: starting after the block's owner; tree: the
half it lies in), so the oracle's result at those positions is exactly what
the full-size call must produce there.  Sample counts are multiples of the
16-byte vector, so the reduced problem's blocks are exactly the samples of
one full-size block each.
"""

import sys

import numpy as np
import torch

from oracle import collectives as C, geometry
from tests.gpu_util import assert_same, to_host


def say(*what):
    print("CASE", *what, flush=True, file=sys.stderr)


def samples(lo, hi, m, rng):
    """m sorted positions in [lo, hi) including both ends (fewer if short)."""
    if hi - lo <= m:
        return np.arange(lo, hi)
    mid = rng.choice(np.arange(lo + 1, hi - 1), size=m - 2, replace=False)
    return np.sort(np.concatenate([[lo, hi - 1], mid]))


def gather(tensors, idx, dt):
    t_idx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    return [to_host(t.index_select(0, t_idx), dt) for t in tensors]


def allreduce_positions(n, count, dt, algo, m, rng):
    """Sampled positions of an all-reduce of `count` elements, `per` in every
    block (ring, one-shot, two-shot: the N blocks; tree: the two halves), or
    None when some block is shorter than `per` (small sizes are compared in
    full instead)."""
    a = geometry.vec_elems(dt)
    per = (m // a) * a
    blocks = geometry.ar_blocks(count, 2 if algo == "tree" else n, dt)
    if any(hi - lo < per for lo, hi in blocks):
        return None
    return np.concatenate([samples(lo, hi, per, rng) for lo, hi in blocks])


def check_allreduce_at(send, recv, n, count, dt, algo, what, chunk=0, m=2048, seed=0):
    """recv (the outputs of an all-reduce of send) equals the oracle at
    sampled positions of every block, bit for bit."""
    idx = allreduce_positions(n, count, dt, algo, m, np.random.default_rng(seed))
    assert idx is not None, f"{what}: blocks shorter than the sample"
    red_in = gather(send, idx, dt)
    want = C.allreduce(red_in, dt, algo, chunk_bytes=chunk or C.DEFAULT_CHUNK_BYTES)
    got = gather(recv, idx, dt)
    for r in range(n):
        assert_same(got[r], want[r], f"{what} rank {r}")


def check_reduce_scatter_at(send, recv, n, rc, dt, algo, what, m=1024, seed=0):
    rng = np.random.default_rng(seed)
    pos = samples(0, rc, m, rng)
    red_in = gather(send, np.concatenate([j * rc + pos for j in range(n)]), dt)
    want = C.reduce_scatter(red_in, dt, algo)
    got = gather(recv, pos, dt)
    for r in range(n):
        assert_same(got[r], want[r], f"{what} rank {r}")


def check_allgather_at(send, recv, n, sc, dt, algo, what, m=1024, seed=0):
    rng = np.random.default_rng(seed)
    pos = samples(0, sc, m, rng)
    red_in = gather(send, pos, dt)
    want = C.allgather(red_in, dt, algo)
    got = gather(recv, np.concatenate([j * sc + pos for j in range(n)]), dt)
    for r in range(n):
        assert_same(got[r], want[r], f"{what} rank {r}")
