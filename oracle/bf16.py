"""bf16 <-> fp32 conversions for the oracle (test infrastructure only).

The all-reduce pages fix the reduction (an elementwise SUM) but not how a
16-bit brain-float payload is added.  Reading taken: a bf16 payload is widened
to fp32 exactly, added in fp32, and rounded back to bf16 with IEEE
round-to-nearest-even.  NaN becomes a quiet NaN that keeps its sign; infinities
and subnormals are kept.

bf16 values are carried as their uint16 bit patterns.
"""

import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact: the 16 bits become the
    high half of the binary32 encoding."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def narrow_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns with round-to-nearest, ties-to-even.

    Textbook integer-bias rounding on the binary32 encoding u: add 0x7FFF plus
    the lowest kept bit, then drop the low 16 bits.  A carry out of the
    mantissa bumps the exponent, which is exactly the rounding of the largest
    finite values up to infinity.  NaNs are made quiet and keep their sign.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    qnan = ((u >> np.uint64(16)) & np.uint64(0x8000)) | np.uint64(0x7FC0)
    return np.where(is_nan, qnan, rounded).astype(np.uint16)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance between two bf16 values on the monotone integer line of their
    encodings (negative values mirrored below zero); +0 and -0 are 0 apart."""

    def key(bits):
        v = np.asarray(bits, dtype=np.uint16).astype(np.int64)
        mag = v & 0x7FFF
        return np.where(v & 0x8000, -mag, mag)

    return np.abs(key(a_bits) - key(b_bits))


def narrow_rne_f64(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns, rounded once to nearest even (no detour
    through fp32, whose own rounding could move a value onto a bf16 tie).
    bf16 keeps 8 significant bits over fp32's exponent range: a value
    m * 2**e (0.5 <= |m| < 1) is rounded to a multiple of 2**(e-8), or of
    2**-133 (the smallest bf16 subnormal) below the normal range."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    _, e = np.frexp(np.where(finite, x, 0.0))
    q = np.maximum(e - 8, -133)
    val = np.ldexp(np.rint(np.ldexp(np.where(finite, x, 0.0), -q)), q)  # rint: half to even
    val = np.where(finite, val, x)
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)  # exact, or +-inf past the largest bf16
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
