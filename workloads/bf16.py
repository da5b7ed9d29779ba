"""bf16 encoding helpers for the seeded input generators.

Inputs are drawn in float32/float64 and rounded once, round-to-nearest-even, to
bfloat16 (1 sign, 8 exponent, 7 mantissa bits).  Both the GPU path (which takes
the raw 16-bit patterns) and the oracle (which takes the exact float64 values of
those patterns) consume the same bits.  This is an encoding, not arithmetic of
the method.
"""
from __future__ import annotations

import numpy as np


def to_bf16_bits(a) -> np.ndarray:
    """Round float values to bf16 (RNE) and return the 16-bit patterns (uint16).

    Rounding is done once from the float64 value (float32 inputs are widened
    exactly first), by adding the RNE bias at bit 45 of the float64 pattern and
    truncating; the result is then exact in float32 and its top 16 bits are the
    bf16 pattern.  Values must be finite and inside the bf16 normal range or
    zero, which every synthetic input here is.
    """
    a = np.asarray(a, dtype=np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bias = np.uint64((1 << 44) - 1) + lsb
    rounded = (bits + bias) & ~np.uint64((1 << 45) - 1)
    f32 = rounded.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 values of bf16 patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_bf16(a) -> np.ndarray:
    """float64 values of round-to-nearest-even bf16(a)."""
    return bf16_bits_to_f64(to_bf16_bits(a))


def to_bf16_bits_f32(a32: np.ndarray) -> np.ndarray:
    """RNE bf16 patterns of a float32 array, chunked to bound memory.

    For float32 input this equals `to_bf16_bits` (float32 -> float64 is exact),
    computed directly on the 32-bit pattern: add 0x7FFF plus the kept LSB.
    """
    a32 = np.ascontiguousarray(a32, dtype=np.float32).reshape(-1)
    out = np.empty(a32.shape, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, a32.size, step):
        u = a32[s:s + step].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[s:s + step] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out
