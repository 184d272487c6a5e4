"""Number-format helpers of the oracle.

* bf16 -> float64 is exact (a bf16 is the upper half of an IEEE binary32).
* float64 -> fp16 rounds once, to nearest with ties to even, straight from binary64 (no
  intermediate binary32 step, which could round twice).  numpy's float64 -> float16 cast does
  exactly this; the pins in tests/test_oracle_numerics.py check it on halfway cases where a
  detour through binary32 would give a different answer, and on subnormals and overflow.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_fp16(x) -> np.ndarray:
    """Round float64 values to fp16 (RNE, single rounding). Returns float16."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def fp16_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).astype(np.float64)
