"""Seeded input tensors (input generation only).

Every value is drawn in float64 from a numpy Generator and stored in the
arithmetic type the workload names. For bfloat16 inputs the value is first
rounded to float32 (IEEE round-to-nearest-even, numpy's cast), then to bfloat16
with round-to-nearest-even on the float32 bit pattern. Both the oracle and the
GPU path read the same stored bits; the float64 view returned next to them is
the exact value of those bits.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) nearest to float32 values, ties to even."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Stored:
    """A tensor as stored for the kernels plus its exact float64 value."""

    def __init__(self, dtype: str, raw: np.ndarray, value: np.ndarray):
        self.dtype = dtype      # "f32" or "bf16"
        self.raw = raw          # float32 array, or uint16 bf16 bits
        self.value = value      # float64, exactly equal to raw

    @property
    def shape(self):
        return self.raw.shape


def store(x64: np.ndarray, dtype: str) -> Stored:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Stored("f32", x32, x32.astype(np.float64))
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Stored("bf16", bits, bf16_bits_to_f64(bits))
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, variance: float = 1.0) -> np.ndarray:
    """float64 draws from N(0, variance); the second parameter is the variance."""
    return rng.standard_normal(shape) * np.sqrt(variance)
