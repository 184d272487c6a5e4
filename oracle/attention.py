"""Attention of the two passes, computed exactly as defined, in float64.

Sources
-------
* VeriCache review, §Prerequisites "Transformer attention and the KV cache": attention is
  softmax(Q K^T / sqrt(d_h)) V; Llama-3.1-8B uses h = 8 KV heads (grouped-query attention).
* Same page, §Draft–Verify Pipeline, steps 2 and 4: the drafter decodes one token per step
  against the compressed cache; the verifier runs one parallel pass over the x drafted positions
  against the full cache, position k conditioned on the drafted tokens before it.

Readings (also in the design notes): query head h reads KV head floor(h / G), G = Hq / Hkv;
scale 1/sqrt(d), no extra terms; verify row i sees the whole context plus drafted rows 0..i
(inclusive, as a decode step sees its own K/V); draft step i uses the same query as verify row i
and sees the compressed context plus drafted rows 0..i.
"""
from __future__ import annotations

import numpy as np


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible=None, spread: bool = False):
    """softmax(q k^T / sqrt(d)) v, rows restricted to ``visible`` keys (bool [rows][keys]).

    Two passes: row maximum over visible scores, then normalised exponential weights.

    With ``spread``, also returns sqrt(sum_t (w_t v_tc)^2) per row and channel, w_t the
    normalised weights.  This is not part of the method: it sizes the parity gates, since an
    implementation whose weights carry independent relative rounding errors of standard deviation
    sigma has an output error of standard deviation at most sigma times this spread."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(d)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    out = (w @ v) / w.sum(axis=1, keepdims=True)
    if not spread:
        return out
    wn = w / w.sum(axis=1, keepdims=True)
    return out, np.sqrt((wn * wn) @ (v * v))


def verify_unit(q: np.ndarray, kctx: np.ndarray, vctx: np.ndarray,
                kblk: np.ndarray, vblk: np.ndarray, spread: bool = False):
    """Verify pass of one (request, layer, kv-head).

    q: [x][G][d] (drafted rows x query heads of the group), kctx/vctx: [n][d] full context,
    kblk/vblk: [>=x][d] drafted rows.  Returns [x][G][d] (and its spread, see ``attention``)."""
    x, G, d = q.shape
    n = kctx.shape[0]
    keys = np.concatenate([kctx, kblk[:x]], axis=0)
    vals = np.concatenate([vctx, vblk[:x]], axis=0)
    row_tok = np.repeat(np.arange(x), G)                      # row (i, j) -> token i
    key_blk = np.arange(n + x) - n                            # <0: context, else block row
    visible = key_blk[None, :] <= row_tok[:, None]
    if spread:
        out, spr = attention(q.reshape(x * G, d), keys, vals, visible, spread=True)
        return out.reshape(x, G, d), spr.reshape(x, G, d)
    out = attention(q.reshape(x * G, d), keys, vals, visible)
    return out.reshape(x, G, d)


def draft_unit(q: np.ndarray, kcomp: np.ndarray, vcomp: np.ndarray,
               kblk: np.ndarray, vblk: np.ndarray, step: int, spread: bool = False):
    """Draft step ``step`` of one (request, layer, kv-head): one query token, G heads.

    q: [G][d]; kcomp/vcomp: [k][d] compressed context (kept rows, or dequantised rows);
    kblk/vblk: drafted rows, of which 0..step are visible.  Returns [G][d] (and its spread, see
    ``attention``)."""
    keys = np.concatenate([kcomp, kblk[:step + 1]], axis=0)
    vals = np.concatenate([vcomp, vblk[:step + 1]], axis=0)
    return attention(q, keys, vals, spread=spread)


def gqa_group(h: int, G: int) -> int:
    """KV head read by query head h."""
    return h // G
