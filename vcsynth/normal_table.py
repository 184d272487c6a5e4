"""Inverse-CDF threshold tables that turn a uniform 32-bit draw into a bf16 normal variate.

For a draw ``u`` in [0, 2**32) the variate is ``RNE_bf16(sigma * Phi^{-1}((u + 0.5) / 2**32))``.
Because ``Phi^{-1}`` and round-to-nearest are both monotone, that is a step function of ``u``:
between two neighbouring bf16 values b_k < b_{k+1} the switch happens at the first ``u`` whose
variate reaches their midpoint, i.e. at ``ceil(Phi(mid / sigma) * 2**32 - 0.5)``.  The table keeps
those switch points (sorted, uint32) and the bf16 value of every non-empty bucket; a lookup is
``values[#{thresholds <= u}]``.  Tails are cut where the quantile of 0.5/2**32 lands (about
6.2 sigma); exact midpoints have probability zero at this resolution and are ignored.

The same table (built once on the host) drives both the numpy generator and the GPU fill kernel,
so both produce identical bits.
"""
from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np
from scipy.special import ndtr


@dataclass(frozen=True)
class NormalTable:
    sigma: float
    thresholds: np.ndarray  # uint32, sorted ascending, len = len(values) - 1
    values_bits: np.ndarray  # uint16 bf16 bit patterns, ascending by value


def _all_bf16_values_in(lo: float, hi: float):
    """Every finite bf16 value in [lo, hi] (no -0), ascending, with its bit pattern."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    ok = np.isfinite(f) & (f >= lo) & (f <= hi) & ~((f == 0) & (bits == 0x8000))
    f = f[ok]
    b = bits[ok].astype(np.uint16)
    order = np.argsort(f, kind="stable")
    return f[order], b[order]


@functools.lru_cache(maxsize=None)
def normal_table(sigma: float) -> NormalTable:
    if not sigma > 0:
        raise ValueError("sigma must be positive")
    vals, bits = _all_bf16_values_in(-8.0 * sigma, 8.0 * sigma)
    mids = 0.5 * (vals[:-1] + vals[1:])  # exact in float64
    thr = np.ceil(ndtr(mids / sigma) * 4294967296.0 - 0.5)
    thr = np.clip(thr, 0.0, 4294967296.0)
    # bucket k spans [lo_k, hi_k); keep the non-empty ones only
    lo = np.concatenate([[0.0], thr])
    hi = np.concatenate([thr, [4294967296.0]])
    keep = hi > lo
    kept_bits = bits[keep]
    kept_lo = lo[keep]
    thresholds = kept_lo[1:].astype(np.uint64)
    assert np.all(thresholds < (1 << 32)) and np.all(np.diff(thresholds.astype(np.int64)) > 0)
    return NormalTable(sigma=float(sigma), thresholds=thresholds.astype(np.uint32),
                       values_bits=np.ascontiguousarray(kept_bits))
