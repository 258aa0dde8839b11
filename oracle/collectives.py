"""The all-reduce family, written out plainly on the CPU (test infrastructure only).

Each function takes a list of N per-rank NumPy arrays (float32, int32, or
uint16 bf16 bit patterns) and returns the N per-rank results.  What the
algorithms compute is an elementwise SUM over ranks; what differs between
them is only the order in which each output element's terms are added and,
for bf16, where the value is rounded back to bf16.  Those orders are fixed
here as follows.

* One-shot all-reduce ("Collective communication: NCCL's algorithms and
  protocols, and custom all-reduce", section "Algorithms", one-shot): every
  rank reads all N inputs and sums them locally.  Reading taken: ascending
  rank order 0..N-1, a left fold, identical on every rank; bf16 rounds once.
* Two-shot all-reduce (same section, two-shot): a reduce-scatter in which
  rank j reads the j-th 1/N slice of every rank and sums it (same order as
  one-shot), then an all-gather in which every rank reads the sums back.
* Ring all-reduce (same section, ring; "NCCL collectives, ring all-reduce &
  launching TP/PP", section "Direct answer": ring = reduce-scatter +
  all-gather): N-1 reduce steps, then N-1 copy steps.  In reduce step s rank r
  sends its partial of block (r-1-s) mod N to rank r+1, which adds its own
  input; in copy step s rank r sends block (r-s) mod N to rank r+1.  Block j's
  sum therefore starts at rank j+1 and ends at rank j, the rank that keeps it
  (reduce-scatter leaves every rank holding just its own share of the sum).  The wire carries
  the payload type, so a bf16 partial is rounded after every hop.
* Tree all-reduce (same section, tree: a double binary tree that reduces
  up the tree and then broadcasts down it, in O(log n) steps).  The page
  gives neither the tree shapes nor how the data is split between the two
  trees.  Reading taken: the buffer is cut in two halves like an N=2 block
  split; half 0 runs on tree 0, half 1 on tree 1.  Both trees are complete
  binary trees in heap layout (position p has children 2p+1 and 2p+2 and
  parent (p-1)/2); tree 0 holds rank p at position p, tree 1 holds rank
  N-1-p, so a rank that is an inner node of one tree is a leaf of the other
  (for even N).  Going up, the node at position p adds, in this order, its
  own input, then the partial of child 2p+1, then that of child 2p+2; it
  sends its partial up rounded to the payload type (the wire carries bf16,
  as on the ring).  The root's sum is the result, and going down every node
  copies its parent's result.
* Reduce-scatter and all-gather ("NCCL collectives...", section "Direct
  answer"): "direct" reads the slices straight from every rank (the
  one-shot / two-shot schedule has a single exchange for these); "ring" runs
  the matching half of the ring.
"""

import numpy as np

from . import dtypes, geometry

DEFAULT_CHUNK_BYTES = 512 * 1024


def _check(inputs, dt):
    dtypes.check(dt)
    n = len(inputs)
    if n < 1:
        raise ValueError("need at least one rank")
    size = len(inputs[0])
    want = np.dtype(dtypes.STORAGE[dt])
    for x in inputs:
        if x.ndim != 1 or len(x) != size or x.dtype != want:
            raise ValueError("every rank needs a 1-D buffer of the same size and type")
    return n, size


def _empty(size, dt):
    return np.zeros(size, dtype=dtypes.STORAGE[dt])


# ----------------------------------------------------------------- all-reduce
def allreduce_oneshot(inputs, dt):
    """Every rank r: out[r] = in[0] + in[1] + ... + in[N-1] (left fold)."""
    n, size = _check(inputs, dt)
    return [dtypes.fold([inputs[i] for i in range(n)], dt) for _ in range(n)]


def allreduce_twoshot(inputs, dt):
    """Reduce-scatter of the N blocks (rank j sums block j over ranks
    0..N-1), then all-gather of the block sums to every rank."""
    n, size = _check(inputs, dt)
    blocks = geometry.ar_blocks(size, n, dt)
    owned = []
    for lo, hi in blocks:  # shot 1: rank j reads block j of every rank
        owned.append(dtypes.fold([inputs[i][lo:hi] for i in range(n)], dt))
    outs = [_empty(size, dt) for _ in range(n)]
    for r in range(n):  # shot 2: every rank reads every block sum back
        for (lo, hi), s in zip(blocks, owned):
            outs[r][lo:hi] = s
    return outs


def _ring_reduce(inputs, blocks, dt, chunk):
    """Reduce-scatter half of the ring.  Returns owned[j] = block j's sum as
    held by rank j after N-1 steps."""
    n = len(inputs)
    biggest = max(hi - lo for lo, hi in blocks) if blocks else 0
    loops = geometry.n_loops(biggest, chunk)
    # partial[r][b] -> list of per-loop payload arrays rank r holds for block b
    partial = [[[None] * loops for _ in range(n)] for _ in range(n)]
    for l in range(loops):
        for s in range(n - 1):
            wire = []
            for r in range(n):  # every rank sends one block per step
                b = (r - 1 - s) % n
                lo, hi = geometry.loop_range(*blocks[b], l, chunk)
                payload = inputs[r][lo:hi] if s == 0 else partial[r][b][l]
                wire.append(((r + 1) % n, b, lo, hi, payload))
            for q, b, lo, hi, payload in wire:  # receiver adds its own input
                partial[q][b][l] = dtypes.add_payloads(payload, inputs[q][lo:hi], dt)
    owned = []
    for j, (lo, hi) in enumerate(blocks):
        if n == 1:
            owned.append(np.array(inputs[0][lo:hi], copy=True))
            continue
        parts = [partial[j][j][l] for l in range(loops)]
        parts = [p for p in parts if p is not None and len(p)]
        owned.append(np.concatenate(parts) if parts else _empty(0, dt))
    return owned


def _ring_gather(owned, blocks, size, dt, chunk):
    """All-gather half of the ring: block j starts at rank j and is copied
    around the ring for N-1 steps."""
    n = len(owned)
    held = [[None] * n for _ in range(n)]  # held[r][b]
    for j in range(n):
        held[j][j] = owned[j]
    biggest = max(hi - lo for lo, hi in blocks) if blocks else 0
    loops = geometry.n_loops(biggest, chunk)
    pieces = [[[None] * loops for _ in range(n)] for _ in range(n)]
    for j in range(n):
        lo, hi = blocks[j]
        for l in range(loops):
            a, b = geometry.loop_range(lo, hi, l, chunk)
            pieces[j][j][l] = owned[j][a - lo:b - lo]
    for l in range(loops):
        for s in range(n - 1):
            wire = []
            for r in range(n):
                b = (r - s) % n
                wire.append(((r + 1) % n, b, pieces[r][b][l]))
            for q, b, payload in wire:
                pieces[q][b][l] = np.array(payload, copy=True)
    outs = [_empty(size, dt) for _ in range(n)]
    for r in range(n):
        for b, (lo, hi) in enumerate(blocks):
            for l in range(loops):
                a, e = geometry.loop_range(lo, hi, l, chunk)
                if e > a:
                    outs[r][a:e] = pieces[r][b][l]
    return outs


def allreduce_ring(inputs, dt, chunk_bytes=DEFAULT_CHUNK_BYTES):
    """Ring all-reduce: N-1 reduce steps then N-1 copy steps, each block
    walked in chunks of `chunk_bytes`."""
    n, size = _check(inputs, dt)
    blocks = geometry.ar_blocks(size, n, dt)
    chunk = geometry.chunk_elems(chunk_bytes, dt)
    owned = _ring_reduce(inputs, blocks, dt, chunk)
    return _ring_gather(owned, blocks, size, dt, chunk)


def tree_rank(n, tree, pos):
    """Rank at heap position `pos` of tree 0 or tree 1."""
    return pos if tree == 0 else n - 1 - pos


def allreduce_tree(inputs, dt):
    """Double binary tree: half h of the buffer is reduced up tree h (children
    before parents; own input, then left child, then right child) and the
    root's sum is broadcast down to every rank."""
    n, size = _check(inputs, dt)
    outs = [_empty(size, dt) for _ in range(n)]
    for tree, (lo, hi) in enumerate(geometry.ar_blocks(size, 2, dt)):
        sent = [None] * n  # what the node at each position sends to its parent
        for pos in reversed(range(n)):
            acc = dtypes.to_acc(inputs[tree_rank(n, tree, pos)][lo:hi], dt)
            for child in (2 * pos + 1, 2 * pos + 2):
                if child < n:
                    acc = dtypes.add(acc, dtypes.to_acc(sent[child], dt), dt)
            sent[pos] = dtypes.from_acc(acc, dt)
        for r in range(n):  # down the tree: every rank ends with the root's sum
            outs[r][lo:hi] = sent[0]
    return outs


ALLREDUCE = {
    "oneshot": allreduce_oneshot,
    "twoshot": allreduce_twoshot,
    "ring": allreduce_ring,
    "tree": allreduce_tree,
}


def allreduce(inputs, dt, algo, chunk_bytes=DEFAULT_CHUNK_BYTES):
    if algo == "ring":
        return allreduce_ring(inputs, dt, chunk_bytes)
    if algo not in ALLREDUCE:
        raise ValueError(f"unknown algorithm {algo!r}")
    return ALLREDUCE[algo](inputs, dt)


# ------------------------------------------------------------ reduce-scatter
def _rs_blocks(inputs, dt):
    n, size = _check(inputs, dt)
    if size % n:
        raise ValueError("reduce-scatter input must hold N * recvcount elements")
    rc = size // n
    return n, rc, [(j * rc, (j + 1) * rc) for j in range(n)]


def reduce_scatter_direct(inputs, dt):
    """Rank r sums slice r of every rank, ranks in ascending order."""
    n, rc, blocks = _rs_blocks(inputs, dt)
    return [dtypes.fold([inputs[i][lo:hi] for i in range(n)], dt) for lo, hi in blocks]


def reduce_scatter_ring(inputs, dt, chunk_bytes=DEFAULT_CHUNK_BYTES):
    """Reduce-scatter half of the ring with blocks of exactly recvcount."""
    n, rc, blocks = _rs_blocks(inputs, dt)
    chunk = geometry.chunk_elems(chunk_bytes, dt)
    return _ring_reduce(inputs, blocks, dt, chunk)


def reduce_scatter(inputs, dt, algo, chunk_bytes=DEFAULT_CHUNK_BYTES):
    if algo in ("oneshot", "twoshot"):
        return reduce_scatter_direct(inputs, dt)
    if algo == "ring":
        return reduce_scatter_ring(inputs, dt, chunk_bytes)
    raise ValueError(f"unknown algorithm {algo!r}")


# ---------------------------------------------------------------- all-gather
def allgather_direct(inputs, dt):
    """Every rank ends with the concatenation in[0] | in[1] | ... | in[N-1]."""
    n, sc = _check(inputs, dt)
    full = np.concatenate([inputs[j] for j in range(n)]) if sc else _empty(0, dt)
    return [np.array(full, copy=True) for _ in range(n)]


def allgather_ring(inputs, dt, chunk_bytes=DEFAULT_CHUNK_BYTES):
    """Copy half of the ring: shard j starts at rank j and walks N-1 hops."""
    n, sc = _check(inputs, dt)
    blocks = [(j * sc, (j + 1) * sc) for j in range(n)]
    chunk = geometry.chunk_elems(chunk_bytes, dt)
    owned = [np.array(inputs[j], copy=True) for j in range(n)]
    return _ring_gather(owned, blocks, n * sc, dt, chunk)


def allgather(inputs, dt, algo, chunk_bytes=DEFAULT_CHUNK_BYTES):
    if algo in ("oneshot", "twoshot"):
        return allgather_direct(inputs, dt)
    if algo == "ring":
        return allgather_ring(inputs, dt, chunk_bytes)
    raise ValueError(f"unknown algorithm {algo!r}")
