"""Helpers shared by the GPU tests: host <-> device buffers and comparisons."""

import numpy as np
import torch

from oracle import bf16

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "bf16":
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(x.copy()).cuda()


def to_host(t: torch.Tensor, dt: str) -> np.ndarray:
    t = t.detach().cpu()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def empty(count: int, dt: str) -> torch.Tensor:
    # Poison so that an element the kernel forgets to write shows up.
    t = torch.empty(count, dtype=TORCH[dt], device="cuda")
    t.view(torch.uint8).fill_(0xA5) if count else None
    return t


def assert_same(got: np.ndarray, want: np.ndarray, what: str):
    """Bit-exact equality (integers, same-order floating point)."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        g, w = got.view(np.uint32), want.view(np.uint32)
    else:
        g, w = got, want
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {bad[:5]}: " \
                          f"got {got[bad[:5]]} want {want[bad[:5]]}"


def widen(x: np.ndarray, dt: str) -> np.ndarray:
    return bf16.widen(x) if dt == "bf16" else x
