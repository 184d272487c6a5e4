"""CPU regeneration of any slice of the synthetic inputs (numpy, bit patterns).

Each function returns exactly the bits the GPU fill kernels write for the same logical
elements, because both evaluate value(seed, stream, logical_index) through the same table.
"""
from __future__ import annotations

import functools

import numpy as np

from . import rng
from .configs import NPOS, XMAX, Config
from .normal_table import normal_table


def _grid(*axes):
    """Broadcastable int64 index grids for the given 1-D axes."""
    out = []
    nd = len(axes)
    for k, a in enumerate(axes):
        shape = [1] * nd
        shape[k] = len(a)
        out.append(np.asarray(a, dtype=np.int64).reshape(shape))
    return out


def q_index(cfg: Config, r, l, i, h, c):
    return (((r * cfg.L + l) * XMAX + i) * cfg.Hq + h) * cfg.d + c


def ctx_index(cfg: Config, r, l, g, p, c):
    return (((r * cfg.L + l) * cfg.Hkv + g) * NPOS + p) * cfg.d + c


def blk_index(cfg: Config, r, l, i, g, c):
    return (((r * cfg.L + l) * XMAX + i) * cfg.Hkv + g) * cfg.d + c


def score_index(cfg: Config, r, l, g, p):
    return ((r * cfg.L + l) * cfg.Hkv + g) * NPOS + p


def q_bits(cfg: Config, r: int, l: int, x: int) -> np.ndarray:
    """Queries of request r, layer l, block rows [0, x): uint16 [x][Hq][d]."""
    i, h, c = _grid(range(x), range(cfg.Hq), range(cfg.d))
    return rng.normal_bf16_bits(cfg.seed, rng.STREAM_Q, q_index(cfg, r, l, i, h, c),
                                normal_table(1.0))


def kctx_bits(cfg: Config, r: int, l: int, g: int, n: int, p0: int = 0) -> np.ndarray:
    """Context keys at positions [p0, p0+n): uint16 [n][d]."""
    p, c = _grid(range(p0, p0 + n), range(cfg.d))
    return rng.normal_bf16_bits(cfg.seed, rng.STREAM_KCTX, ctx_index(cfg, r, l, g, p, c),
                                normal_table(1.0))


def vctx_bits(cfg: Config, r: int, l: int, g: int, n: int, p0: int = 0) -> np.ndarray:
    p, c = _grid(range(p0, p0 + n), range(cfg.d))
    return rng.normal_bf16_bits(cfg.seed, rng.STREAM_VCTX, ctx_index(cfg, r, l, g, p, c),
                                normal_table(1.0))


def kblk_bits(cfg: Config, r: int, l: int, g: int, x: int) -> np.ndarray:
    """Drafted-block keys, rows [0, x): uint16 [x][d]."""
    i, c = _grid(range(x), range(cfg.d))
    return rng.normal_bf16_bits(cfg.seed, rng.STREAM_KBLK, blk_index(cfg, r, l, i, g, c),
                                normal_table(1.0))


def vblk_bits(cfg: Config, r: int, l: int, g: int, x: int) -> np.ndarray:
    i, c = _grid(range(x), range(cfg.d))
    return rng.normal_bf16_bits(cfg.seed, rng.STREAM_VBLK, blk_index(cfg, r, l, i, g, c),
                                normal_table(1.0))


def scores_u32(cfg: Config, r: int, l: int, g: int, n: int) -> np.ndarray:
    """Per-position token scores (uint32, larger = keep first) for positions [0, n)."""
    p = np.arange(n, dtype=np.int64)
    return rng.u32(cfg.seed, rng.STREAM_SCORE, score_index(cfg, r, l, g, p))


@functools.lru_cache(maxsize=4)
def _wu_cached(seed: int, width: int, vocab: int, sigma: float) -> np.ndarray:
    w, v = _grid(range(width), range(vocab))
    return rng.normal_bf16_bits(seed, rng.STREAM_WU, w * vocab + v, normal_table(sigma))


def wu_bits(cfg: Config) -> np.ndarray:
    """LM-head stand-in W_u: uint16 [width][vocab], N(0, 1/width)."""
    return _wu_cached(cfg.seed, cfg.wu_width, cfg.vocab, cfg.wu_sigma)
