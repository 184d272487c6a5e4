"""Compressed KV cache of the drafter: token dropping and KIVI-style quantisation (fp64).

Sources
-------
* VeriCache review, §Prerequisites "KV cache compression: lossy by construction": token dropping
  keeps a subset of positions per layer/head; quantisation lowers the bits per element (KIVI,
  2-bit).
* Same page, §Compression Method Integration, the CompressedKV record and "Scope and current
  limitations": heads of a layer may drop different positions but keep the same count; the bit
  scheme is uniform.
* KVBoost summary page, §1 and §2: KIVI-style asymmetric quantisation is per-channel for keys
  and per-token for values.

Readings where the pages are silent (each also listed in the design notes):
* Kept set = the most recent R positions plus the top-m of the older positions by a seeded
  per-head score (larger first, ties to the lower position), returned in ascending order.
* Quantiser: asymmetric min-max over groups of 32: keys per channel over 32 consecutive tokens
  of the stored sequence, values per token over 32 consecutive channels.  Per group
  scale = fp16(round((max - min) / (2^b - 1))), zero = fp16(round(min)) with single RNE rounding
  from float64; code = clamp(rint_half_even((x - zero) / scale), 0, 2^b - 1), code = 0 when the
  scale is 0; dequantised value = code * scale + zero.  A short last key group uses its actual
  members.  For drop + quantise the stored sequence is the kept tokens in ascending position
  order.
"""
from __future__ import annotations

import numpy as np

from .numerics import f64_to_fp16, fp16_to_f64

GROUP = 32


def kept_positions(scores: np.ndarray, n: int, recent: int, top: int) -> np.ndarray:
    """Kept positions of one (request, layer, kv-head): recent window plus top-scored older ones.

    ``scores`` holds one unsigned score per position [0, n).  Returns int64, ascending, unique,
    of length min(n, recent + top)."""
    if not 0 <= recent:
        raise ValueError("recent must be >= 0")
    recent = min(recent, n)
    older = n - recent
    top = min(top, older)
    pos = np.arange(older, dtype=np.int64)
    sc = np.asarray(scores[:older]).astype(np.int64)
    # primary key: score descending; secondary: position ascending
    order = np.lexsort((pos, -sc))
    chosen = pos[order[:top]]
    kept = np.concatenate([np.sort(chosen), np.arange(older, n, dtype=np.int64)])
    return kept


def _group_params(mn: np.ndarray, mx: np.ndarray, bits: int):
    levels = (1 << bits) - 1
    scale = f64_to_fp16((mx - mn) / levels)
    zero = f64_to_fp16(mn)
    return scale, zero


def _codes(x: np.ndarray, scale16: np.ndarray, zero16: np.ndarray, bits: int) -> np.ndarray:
    levels = (1 << bits) - 1
    s = fp16_to_f64(scale16)
    z = fp16_to_f64(zero16)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((x - z) / s)  # numpy rint: round half to even
    c = np.where(s == 0, 0.0, c)
    return np.clip(c, 0, levels).astype(np.uint8)


def quantize_keys(k: np.ndarray, bits: int):
    """Per-channel key quantisation over groups of 32 consecutive stored tokens.

    k: float64 [T][d].  Returns (codes uint8 [T][d], scale fp16 [ngroups][d], zero fp16 [ngroups][d]).
    """
    T, d = k.shape
    ng = (T + GROUP - 1) // GROUP
    codes = np.zeros((T, d), dtype=np.uint8)
    scale = np.zeros((ng, d), dtype=np.float16)
    zero = np.zeros((ng, d), dtype=np.float16)
    for gi in range(ng):
        blk = k[gi * GROUP:(gi + 1) * GROUP]
        s, z = _group_params(blk.min(axis=0), blk.max(axis=0), bits)
        scale[gi], zero[gi] = s, z
        codes[gi * GROUP:(gi + 1) * GROUP] = _codes(blk, s[None, :], z[None, :], bits)
    return codes, scale, zero


def quantize_values(v: np.ndarray, bits: int):
    """Per-token value quantisation over groups of 32 consecutive channels.

    v: float64 [T][d] with d a multiple of 32.  Returns (codes uint8 [T][d],
    scale fp16 [T][d/32], zero fp16 [T][d/32])."""
    T, d = v.shape
    if d % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    vg = v.reshape(T, d // GROUP, GROUP)
    s, z = _group_params(vg.min(axis=2), vg.max(axis=2), bits)
    codes = _codes(vg, s[:, :, None], z[:, :, None], bits).reshape(T, d)
    return codes, s, z


def dequantize_keys(codes, scale, zero) -> np.ndarray:
    T, d = codes.shape
    grp = np.arange(T) // GROUP
    return codes.astype(np.float64) * fp16_to_f64(scale)[grp] + fp16_to_f64(zero)[grp]


def dequantize_values(codes, scale, zero) -> np.ndarray:
    T, d = codes.shape
    ch = np.arange(d) // GROUP
    return codes.astype(np.float64) * fp16_to_f64(scale)[:, ch] + fp16_to_f64(zero)[:, ch]
