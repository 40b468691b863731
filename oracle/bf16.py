"""Oracle: rounding of a float64 value to the nearest bfloat16 (test infrastructure).

bfloat16 keeps the float32 sign and exponent and 7 explicit mantissa bits.
Rounding is to nearest, ties to even, applied directly to the float64 value
(52 mantissa bits -> 7), for finite values in the normal float32 range.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    b = x.view(np.uint64)
    drop = 52 - 7
    keep_lsb = (b >> np.uint64(drop)) & np.uint64(1)
    half = np.uint64((1 << (drop - 1)) - 1)
    r = (b + half + keep_lsb) & ~np.uint64((1 << drop) - 1)
    return r.view(np.float64)
