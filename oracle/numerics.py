"""Storage-format conversions for the oracle (test infrastructure only).

bfloat16 has a sign bit, 8 exponent bits (bias 127, same range as float32) and
7 stored fraction bits, i.e. 8 significant bits for normal numbers; its
subnormals are spaced 2**-133.  Rounding here is IEEE round-to-nearest with
ties to even, applied ONCE, straight from float64.  (Going float64 -> float32 ->
bfloat16 would round twice and can differ.)
"""
from __future__ import annotations

import numpy as np

BF16_MIN_NORMAL_EXP = -126   # smallest normal bfloat16 is 2**-126
BF16_SUBNORMAL_QUANTUM_EXP = -133
BF16_SIGNIFICANT_BITS = 8


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), once.

    Returns float64 values that are exactly representable in bfloat16.
    A value x = m * 2**e with 0.5 <= |m| < 1 keeps 8 significant bits, so its
    rounding quantum is 2**(e - 8); below 2**-126 the quantum is fixed at 2**-133.
    np.rint rounds half to even, and scaling by a power of two is exact, so the
    result is the correctly rounded value.  Magnitudes at or above the overflow
    threshold become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_f64_to_bf16: non-finite input")
    _, e = np.frexp(x)
    q = np.maximum(e - BF16_SIGNIFICANT_BITS, BF16_SUBNORMAL_QUANTUM_EXP)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, y), y)
    return y


def f64_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of round_f64_to_bf16(x)."""
    y = round_f64_to_bf16(x)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)       # exact: y has at most 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_f64_to_f32(x) -> np.ndarray:
    """Round float64 to float32 (ties to even) and return it widened back to float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_storage(x, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage dtype ("bf16" or "f32"); float64 result."""
    if dtype == "bf16":
        return round_f64_to_bf16(x)
    if dtype == "f32":
        return round_f64_to_f32(x)
    raise ValueError(dtype)


def significant_bits(dtype: str) -> int:
    return {"bf16": 8, "f32": 24}[dtype]
