"""Payload types and the SUM the collectives apply (test infrastructure only).

The collectives on the pages combine tensors by summing ("NCCL collectives,
ring all-reduce & launching TP/PP", section "Direct answer": all-reduce
combines (sums) a tensor every GPU holds).  Three payload types are covered:

* ``f32``  binary32; each add is one IEEE round-to-nearest-even add.
* ``i32``  two's-complement 32-bit; adds wrap.
* ``bf16`` carried as uint16 bit patterns; widened to fp32 for the add and
  rounded back to bf16 (see ``oracle.bf16``) where the schedule puts a bf16
  value on the wire or into an output buffer.
"""

import numpy as np

from . import bf16

DTYPES = ("f32", "bf16", "i32")
ESIZE = {"f32": 4, "bf16": 2, "i32": 4}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}


def check(dt: str) -> None:
    if dt not in ESIZE:
        raise ValueError(f"unknown payload type {dt!r}")


def to_acc(x: np.ndarray, dt: str) -> np.ndarray:
    """Payload -> accumulator (fp32 for f32/bf16, int32 for i32), exact."""
    check(dt)
    if dt == "bf16":
        return bf16.widen(x)
    return np.array(x, dtype=STORAGE[dt], copy=True)


def add(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    """One elementwise add of two accumulators: fp32 RNE or int32 wrap."""
    check(dt)
    if dt == "i32":
        return np.add(a.astype(np.int32), b.astype(np.int32), dtype=np.int32)
    return np.add(a.astype(np.float32), b.astype(np.float32), dtype=np.float32)


def from_acc(acc: np.ndarray, dt: str) -> np.ndarray:
    """Accumulator -> payload (bf16 rounds to nearest even; others exact)."""
    check(dt)
    if dt == "bf16":
        return bf16.narrow_rne(acc)
    return np.array(acc, dtype=STORAGE[dt], copy=True)


def fold(values, dt: str) -> np.ndarray:
    """Left fold of a sequence of payload arrays in the given order, in the
    accumulator type, rounded to the payload type once at the end."""
    it = iter(values)
    acc = to_acc(next(it), dt)
    for v in it:
        acc = add(acc, to_acc(v, dt), dt)
    return from_acc(acc, dt)


def add_payloads(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    """One ring hop: two payloads widened, added, rounded back to payload."""
    return from_acc(add(to_acc(a, dt), to_acc(b, dt), dt), dt)
