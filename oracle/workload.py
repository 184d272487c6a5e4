"""One (request, layer) instance of a workload, end to end, from the seeded inputs.

Follows the per-request cycle of the VeriCache review (§Draft–Verify Pipeline): the drafter's
cache is the compressed context (§Compression Method Integration, CompressedKV), x draft steps
each attend over it plus the drafted rows so far, the verifier attends over the full context
plus the drafted rows causally, both outputs go through the LM-head stand-in, and the greedy
accept compares their argmax tokens.

Inputs come from ``vcsynth`` (the shared seeded generator); everything computed here is the
oracle's own float64 arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from vcsynth import configs as C
from vcsynth import tensors as T

from . import accept as acc
from . import attention as att
from . import compress as cmp
from .numerics import bf16_to_f64


@dataclass
class Compressed:
    """Drafting cache of one (request, layer, kv-head) in float64, plus what produced it."""
    k: np.ndarray                      # [k_r][d] keys the drafter attends over
    v: np.ndarray                      # [k_r][d]
    kept: Optional[np.ndarray] = None  # kept positions (drop kinds)
    kcodes: Optional[np.ndarray] = None
    kscale: Optional[np.ndarray] = None
    kzero: Optional[np.ndarray] = None
    vcodes: Optional[np.ndarray] = None
    vscale: Optional[np.ndarray] = None
    vzero: Optional[np.ndarray] = None


def context(cfg: C.Config, r: int, l: int, g: int):
    n = cfg.reqs[r].ctx_len
    return (bf16_to_f64(T.kctx_bits(cfg, r, l, g, n)),
            bf16_to_f64(T.vctx_bits(cfg, r, l, g, n)))


def block(cfg: C.Config, r: int, l: int, g: int, x: int):
    return (bf16_to_f64(T.kblk_bits(cfg, r, l, g, x)),
            bf16_to_f64(T.vblk_bits(cfg, r, l, g, x)))


def compressed(cfg: C.Config, r: int, l: int, g: int, kctx=None, vctx=None) -> Compressed:
    """The drafter's cache for one kv head under the request's compression setting."""
    req = cfg.reqs[r]
    if kctx is None:
        kctx, vctx = context(cfg, r, l, g)
    n = req.ctx_len
    if req.comp in (C.COMP_DROP, C.COMP_DROP_KIVI4):
        kept = cmp.kept_positions(T.scores_u32(cfg, r, l, g, n), n, req.recent, req.top)
        ks, vs = kctx[kept], vctx[kept]
    else:
        kept = None
        ks, vs = kctx, vctx
    if req.comp == C.COMP_DROP:
        return Compressed(k=ks, v=vs, kept=kept)
    bits = req.bits
    kc, ksc, kz = cmp.quantize_keys(ks, bits)
    vc, vsc, vz = cmp.quantize_values(vs, bits)
    return Compressed(k=cmp.dequantize_keys(kc, ksc, kz), v=cmp.dequantize_values(vc, vsc, vz),
                      kept=kept, kcodes=kc, kscale=ksc, kzero=kz, vcodes=vc, vscale=vsc, vzero=vz)


def queries(cfg: C.Config, r: int, l: int, x: int) -> np.ndarray:
    """[x][Hq][d] float64."""
    return bf16_to_f64(T.q_bits(cfg, r, l, x))


def verify_out(cfg: C.Config, r: int, l: int, g: Optional[int] = None, x: Optional[int] = None,
               spread: bool = False):
    """Verify output [x][Hq][d] (or [x][G][d] for one kv head g); with ``spread``, also the
    weight spread of every output element (see ``attention.attention``)."""
    x = cfg.reqs[r].x if x is None else x
    q = queries(cfg, r, l, x)
    G = cfg.G
    heads = range(cfg.Hkv) if g is None else [g]
    outs, sprs = [], []
    for gg in heads:
        kc, vc = context(cfg, r, l, gg)
        kb, vb = block(cfg, r, l, gg, x)
        res = att.verify_unit(q[:, gg * G:(gg + 1) * G], kc, vc, kb, vb, spread=spread)
        outs.append(res[0] if spread else res)
        if spread:
            sprs.append(res[1])
    out = np.concatenate(outs, axis=1)
    return (out, np.concatenate(sprs, axis=1)) if spread else out


def draft_out(cfg: C.Config, r: int, l: int, steps, g: Optional[int] = None, comp_cache=None,
              spread: bool = False):
    """Draft outputs for the given steps: [len(steps)][Hq][d] (or [..][G][d] for kv head g);
    with ``spread``, also the weight spread of every output element."""
    steps = list(steps)
    xmax = max(steps) + 1
    q = queries(cfg, r, l, xmax)
    G = cfg.G
    heads = range(cfg.Hkv) if g is None else [g]
    out = np.zeros((len(steps), G * len(heads), cfg.d))
    spr = np.zeros_like(out)
    for hi, gg in enumerate(heads):
        cm = comp_cache[gg] if comp_cache is not None else compressed(cfg, r, l, gg)
        kb, vb = block(cfg, r, l, gg, xmax)
        for si, i in enumerate(steps):
            res = att.draft_unit(q[i, gg * G:(gg + 1) * G], cm.k, cm.v, kb, vb, i, spread=spread)
            if spread:
                out[si, hi * G:(hi + 1) * G], spr[si, hi * G:(hi + 1) * G] = res
            else:
                out[si, hi * G:(hi + 1) * G] = res
    return (out, spr) if spread else out


@dataclass
class RoundResult:
    verify_o: np.ndarray     # [x][Hq][d]
    draft_o: np.ndarray      # [x][Hq][d]
    verify_logits: np.ndarray
    draft_logits: np.ndarray
    verify_tok: np.ndarray
    draft_tok: np.ndarray
    verify_gap: np.ndarray
    draft_gap: np.ndarray
    accept_len: int
    next_tok: int
    flagged: bool
    verify_spread: Optional[np.ndarray] = None   # weight spreads (``attention.attention``)
    draft_spread: Optional[np.ndarray] = None


def round_instance(cfg: C.Config, r: int, l: int, spread: bool = False) -> RoundResult:
    """One draft-verify round of instance (r, l): x draft steps, verify, logits, accept."""
    x = cfg.reqs[r].x
    vs = ds = None
    if spread:
        vo, vs = verify_out(cfg, r, l, spread=True)
        do, ds = draft_out(cfg, r, l, range(x), spread=True)
    else:
        vo = verify_out(cfg, r, l)
        do = draft_out(cfg, r, l, range(x))
    wu = bf16_to_f64(T.wu_bits(cfg))
    zv = acc.logits(vo.reshape(x, -1), wu)
    zd = acc.logits(do.reshape(x, -1), wu)
    tv, gv = acc.argmax_gap(zv)
    td, gd = acc.argmax_gap(zd)
    a, nxt = acc.accept(td, tv)
    return RoundResult(vo, do, zv, zd, tv, td, gv, gd, a, nxt,
                       acc.accept_flagged(a, x, gd, gv), vs, ds)
