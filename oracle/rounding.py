"""Rounding helpers of the oracle (test infrastructure only).

* ``bf16_rne``  -- round float32 values to the nearest bfloat16 value, ties to
  even, by bit manipulation of the float32 encoding (bfloat16 is the top 16
  bits of a float32).
* ``f16_rne``   -- round float32 values to the nearest float16 value, ties to
  even (numpy's float32 -> float16 conversion is IEEE round-to-nearest-even).
* ``exact_sum`` -- the fp64 value nearest to the exact sum of a vector
  (``math.fsum`` returns the correctly rounded sum, so the result does not
  depend on summation order).
"""

from __future__ import annotations

import math

import numpy as np


def bf16_rne(x) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def f16_rne(x) -> np.ndarray:
    """float32 -> nearest float16 (ties to even), returned as float32 values."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float32 values to the 16-bit input dtype ("f16" or "bf16")."""
    if dtype == "bf16":
        return bf16_rne(x)
    if dtype == "f16":
        return f16_rne(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def exact_sum(vec) -> float:
    """Correctly rounded fp64 value of the exact sum of ``vec``."""
    return math.fsum(np.asarray(vec, dtype=np.float64).tolist())


def exact_sums_rows(mat) -> np.ndarray:
    """``exact_sum`` of every row of a 2-D array."""
    mat = np.asarray(mat, dtype=np.float64)
    return np.array([math.fsum(r) for r in mat.tolist()], dtype=np.float64)
