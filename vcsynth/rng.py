"""Counter-based seeded generator for the synthetic workloads (CPU side).

Every value is a pure function of (seed, stream, logical index), so any element of any
tensor can be regenerated on its own, independent of the memory layout it ends up in.

* ``u64(seed, stream, idx)`` is output number ``idx + 1`` of a SplitMix64 sequence whose
  state starts at ``key(seed, stream)``; SplitMix64 is Steele, Lea and Flood's generator
  ("Fast splittable pseudorandom number generators", OOPSLA 2014): the state advances by the
  odd constant GAMMA and each output is the state passed through the 64-bit finaliser ``mix64``.
* ``u32`` is the upper half of ``u64``.
* Normal variates use inverse-CDF sampling rounded to bf16: ``u32`` selects a bucket of a
  threshold table built from the normal CDF (see :mod:`vcsynth.normal_table`), so the result
  is a table lookup, identical on any machine that uses the same table.

This module holds no attention, compression or accept arithmetic: it only draws numbers.
The GPU fill kernels in ``vcsynth/csrc/synth.hip`` implement the same definition.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

# Stream ids: one per kind of random input.
STREAM_Q = 1
STREAM_KCTX = 2
STREAM_VCTX = 3
STREAM_KBLK = 4
STREAM_VBLK = 5
STREAM_WU = 6
STREAM_SCORE = 7
STREAM_DRAWS = 8
STREAM_PAGEPERM = 9
STREAM_UDRAFT = 10     # uniforms of the drafter's sampling (temperature > 0)
STREAM_UACC = 11       # uniforms of the keep test
STREAM_URES = 12       # uniforms of the residual / bonus draw

_S30 = np.uint64(30)
_S27 = np.uint64(27)
_S31 = np.uint64(31)
_S32 = np.uint64(32)


def mix64(z):
    """SplitMix64 output finaliser on uint64 (array or scalar); arithmetic wraps mod 2**64."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _S30)) * M1
        z = (z ^ (z >> _S27)) * M2
    return z ^ (z >> _S31)


def stream_key(seed: int, stream: int) -> np.uint64:
    """Starting SplitMix64 state for one (seed, stream) pair."""
    with np.errstate(over="ignore"):
        s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) * GAMMA + np.uint64(stream)
    return np.uint64(mix64(s))


def u64(seed: int, stream: int, idx) -> np.ndarray:
    """64-bit draw number ``idx`` (0-based) of stream ``stream`` under ``seed``."""
    key = stream_key(seed, stream)
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = key + (i + np.uint64(1)) * GAMMA
    return mix64(state)


def u32(seed: int, stream: int, idx) -> np.ndarray:
    """Upper 32 bits of :func:`u64`, as uint32."""
    return (u64(seed, stream, idx) >> _S32).astype(np.uint32)


def uniform01(seed: int, stream: int, idx) -> np.ndarray:
    """(u32 + 0.5) / 2**32 in float64: strictly inside (0, 1)."""
    return (u32(seed, stream, idx).astype(np.float64) + 0.5) / 4294967296.0


_BUCKET_BITS = 20
_buckets = {}


def _bucket_bounds(table):
    """For each of the 2**20 buckets of the top bits of u, the bucket index ``#{thresholds <= u}``
    at the bucket's first and last u.  The count is monotone in u, so where the two agree every
    u of the bucket has that index."""
    hit = _buckets.get(id(table))
    if hit is not None and hit[0] is table:
        return hit[1], hit[2]
    first = np.arange(1 << _BUCKET_BITS, dtype=np.uint64) << np.uint64(32 - _BUCKET_BITS)
    last = first + np.uint64((1 << (32 - _BUCKET_BITS)) - 1)
    th = table.thresholds.astype(np.uint64)
    lo = np.searchsorted(th, first, side="right").astype(np.int32)
    hi = np.searchsorted(th, last, side="right").astype(np.int32)
    _buckets[id(table)] = (table, lo, hi)
    return lo, hi


def normal_bf16_bits(seed: int, stream: int, idx, table) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma^2) draws, sigma fixed by ``table``: the value of
    bucket ``#{thresholds <= u}``.  The count is read from a per-bucket table of the top bits of
    u, and searched among the thresholds only where a bucket holds one."""
    u = np.asarray(u32(seed, stream, idx))
    return table.values_bits[bucket_of(table, u.reshape(-1))].reshape(u.shape)


def bucket_of(table, u: np.ndarray) -> np.ndarray:
    """``#{thresholds <= u}`` for a 1-D uint32 array u (the same as a right-sided search)."""
    lo, hi = _bucket_bounds(table)
    b = u >> np.uint32(32 - _BUCKET_BITS)
    k = lo[b]
    amb = hi[b] != k
    if amb.any():
        k[amb] = np.searchsorted(table.thresholds, u[amb], side="right")
    return k


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact bf16 -> float64 conversion of uint16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
