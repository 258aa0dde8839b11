"""Block and chunk geometry of the schedules (test infrastructure only).

Two-shot and ring split each rank's buffer into N blocks, one per rank
("Collective communication: NCCL's algorithms and protocols, and custom
all-reduce", section "Algorithms": two-shot reads 1/n of the other GPUs' data;
ring moves (n-1)/n of the message in each phase).  The pages do not say where
the block boundaries fall when N does not divide the element count.  Reading
taken: every block but the last holds B elements, where B is ceil(count / N)
rounded up to a whole 16-byte vector (4 fp32/int32 or 8 bf16 elements), so
every block starts on a 16-byte boundary; the trailing blocks may be short or
empty.  Reduce-scatter and all-gather use blocks of exactly the per-rank
receive / send count.

The ring pipelines each block in chunks ("NCCL collectives, ring all-reduce &
launching TP/PP", section "Deep dive": the ring pipelines the data in chunks
so every link is busy).  Loop l covers elements [l*C, (l+1)*C) of every block,
clipped to the block.
"""

from .dtypes import ESIZE


def vec_elems(dt: str) -> int:
    """Elements per 16-byte vector."""
    return 16 // ESIZE[dt]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def ar_block_elems(count: int, nranks: int, dt: str) -> int:
    """All-reduce block size B in elements (see the module docstring)."""
    if nranks < 1:
        raise ValueError("nranks must be >= 1")
    a = vec_elems(dt)
    return ceil_div(ceil_div(count, nranks), a) * a


def block_range(j: int, block: int, total: int):
    """[lo, hi) of block j when blocks hold `block` elements of `total`."""
    lo = min(j * block, total)
    hi = min((j + 1) * block, total)
    return lo, hi


def ar_blocks(count: int, nranks: int, dt: str):
    """The N all-reduce blocks as a list of (lo, hi)."""
    b = ar_block_elems(count, nranks, dt)
    return [block_range(j, b, count) for j in range(nranks)]


def chunk_elems(chunk_bytes: int, dt: str) -> int:
    """Chunk size in elements; at least one 16-byte vector."""
    if chunk_bytes <= 0:
        raise ValueError("chunk_bytes must be positive")
    a = vec_elems(dt)
    return max(a, (chunk_bytes // ESIZE[dt]) // a * a)


def n_loops(block: int, chunk: int) -> int:
    """Number of chunk loops needed to cover the largest block."""
    return ceil_div(block, chunk) if block > 0 else 0


def loop_range(lo: int, hi: int, loop: int, chunk: int):
    """[a, b) of loop `loop` inside block [lo, hi), possibly empty."""
    a = min(lo + loop * chunk, hi)
    b = min(lo + (loop + 1) * chunk, hi)
    return a, b
