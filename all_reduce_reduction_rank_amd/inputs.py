"""Seeded synthetic rank buffers.

This module only draws random numbers; it holds none of the collectives'
arithmetic.  Both the HIP path's tests and the CPU oracle consume what it
returns.

Rank r of a workload draws from ``numpy.random.default_rng([seed, cfg, N, r])``
so every rank's buffer is reproducible on its own.  Distributions:

``uniform``     fp32 uniform on [-1, 1)
``normal``      N(0, 1)
``normal_1e-3`` N(0, sigma = 1e-3)   (gradient buckets)
``int20``       int32 uniform on [-2**20, 2**20]
``ones``        every element 1

A bf16 buffer holds the fp32 draws converted by torch (nearest bf16, ties to
even: a library conversion, not arithmetic of this module); it is returned
as the uint16 bit patterns.
"""

import numpy as np

DISTS = ("uniform", "normal", "normal_1e-3", "int20", "ones")
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}


def rank_rng(seed: int, cfg: int, nranks: int, rank: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, nranks, rank])


def _draw(rng, size, dt, dist):
    if dist == "ones":
        if dt == "bf16":
            return np.full(size, 0x3F80, dtype=np.uint16)
        return np.ones(size, dtype=_STORAGE[dt])
    if dist == "int20":
        v = rng.integers(-(2 ** 20), 2 ** 20, size=size, endpoint=True)
        if dt == "i32":
            return v.astype(np.int32)
        f = v.astype(np.float32)
    elif dist == "uniform":
        f = rng.uniform(-1.0, 1.0, size=size).astype(np.float32)
    elif dist == "normal":
        f = rng.standard_normal(size=size, dtype=np.float32)
    elif dist == "normal_1e-3":
        f = (rng.standard_normal(size=size, dtype=np.float32) * np.float32(1e-3)).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if dt == "f32":
        return f
    if dt == "bf16":  # torch's conversion: nearest bf16, ties to even
        import torch

        return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dt == "i32":
        return np.rint(f * 1024).astype(np.int32)
    raise ValueError(f"unknown payload type {dt!r}")


def rank_inputs(nranks: int, count: int, dt: str, dist: str, seed: int = 0, cfg: int = 0):
    """N host arrays of `count` elements each (uint16 bit patterns for bf16)."""
    if dt not in _STORAGE:
        raise ValueError(f"unknown payload type {dt!r}")
    return [_draw(rank_rng(seed, cfg, nranks, r), count, dt, dist) for r in range(nranks)]


def device_rank_inputs(nranks: int, count: int, dt: str, dist: str, seed: int = 0, cfg: int = 0,
                       device: str = "cuda"):
    """N device tensors drawn on the GPU with torch's seeded generator (for
    buffers too large to draw on the host).  Same distributions as
    `rank_inputs`, a different (torch) stream of random numbers."""
    import torch

    out = []
    for r in range(nranks):
        g = torch.Generator(device=device)
        g.manual_seed((((seed * 1000003 + cfg) * 1000003 + nranks) * 1000003 + r) % (2 ** 63 - 1))
        if dist == "ones":
            t = torch.ones(count, dtype=torch.float32, device=device)
        elif dist == "int20":
            t = torch.randint(-(2 ** 20), 2 ** 20 + 1, (count,), generator=g, device=device, dtype=torch.int64)
            if dt == "i32":
                out.append(t.to(torch.int32))
                continue
            t = t.to(torch.float32)
        elif dist == "uniform":
            t = torch.rand(count, generator=g, device=device, dtype=torch.float32) * 2 - 1
        elif dist == "normal":
            t = torch.randn(count, generator=g, device=device, dtype=torch.float32)
        elif dist == "normal_1e-3":
            t = torch.randn(count, generator=g, device=device, dtype=torch.float32) * 1e-3
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        if dt == "f32":
            out.append(t)
        elif dt == "bf16":  # nearest bf16, ties to even, as for the host generator
            out.append(t.to(torch.bfloat16))
        else:
            out.append(torch.round(t * 1024).to(torch.int32))
    return out
