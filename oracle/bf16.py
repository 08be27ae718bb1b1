"""bf16 <-> fp32 by bit manipulation.  TEST INFRASTRUCTURE ONLY.

The README's API guide stores hidden states and weights as bf16.  bf16 is the
upper 16 bits of an IEEE fp32; narrowing uses round-to-nearest-even (the
rounding of torch's conversion and of gfx950's packed bf16 convert).  NaN does
not occur in these workloads and is rejected.
"""
import numpy as np


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN has no defined bf16 rounding here")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest) -> bf16 (nearest even)."""
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))
