"""Greedy accept of a drafted block (float64 / integer).

Source: VeriCache review, §Draft–Verify Pipeline, steps 5 and 6 and the per-request cycle:
walk the drafted tokens; at the first position where the drafted token differs from the
verifier's prediction, accept the drafted tokens before it plus the verifier's token there;
if every drafted token matches, accept all of them plus the verifier's bonus prediction.

Reading (0-based): verify row i and draft step i predict the same slot.  The accept length
a = min{i < x : draft[i] != verify[i]}, or x when all match; the next token is verify[a] when
the verifier produced a row a (a < x, or a == x with a bonus row, x_v = x + 1), else -1.
Argmax ties resolve to the smallest token id.  A row is "near-tie" when its top-2 logit gap is
below 1e-3; an accept length is flagged when any row it depends on is near-tie on either side.
"""
from __future__ import annotations

import numpy as np

TIE_GAP = 1e-3


def argmax_gap(logits: np.ndarray):
    """Per row: (argmax with lowest-index ties, top1 - top2 gap). logits [..., V]."""
    z = np.asarray(logits, dtype=np.float64)
    t = np.argmax(z, axis=-1)  # numpy returns the first maximal index
    top1 = np.take_along_axis(z, t[..., None], axis=-1)[..., 0]
    rest = z.copy()
    np.put_along_axis(rest, t[..., None], -np.inf, axis=-1)
    gap = top1 - rest.max(axis=-1)
    return t.astype(np.int64), gap


def accept(draft_tok, verify_tok):
    """(accept length a, next token) for one drafted block.

    draft_tok: x drafted tokens; verify_tok: x or x + 1 verifier predictions."""
    x = len(draft_tok)
    if len(verify_tok) not in (x, x + 1):
        raise ValueError("verifier must give x or x + 1 predictions")
    a = x
    for i in range(x):
        if draft_tok[i] != verify_tok[i]:
            a = i
            break
    nxt = int(verify_tok[a]) if a < len(verify_tok) else -1
    return a, nxt


def accept_block(draft_tok, verify_tok):
    """(accept length a, next token) when the verifier may have given fewer rows than drafted
    slots.  Reading: a drafted slot without a verifier row cannot be checked, so the block ends at
    the verifier's last row and the rule above runs on the first len(verify_tok) drafted slots
    (then a <= len(verify_tok) and next is -1 when every compared slot matched)."""
    if len(verify_tok) < len(draft_tok):
        return accept(list(draft_tok)[: len(verify_tok)], verify_tok)
    return accept(draft_tok, verify_tok)


def accept_flagged(a: int, x: int, draft_gap, verify_gap, tie_gap: float = TIE_GAP) -> bool:
    """True if the accept length depends on a near-tie row (rows 0..min(a, x-1))."""
    last = min(a, x - 1)
    dg = np.asarray(draft_gap)[: last + 1]
    vg = np.asarray(verify_gap)[: last + 1]
    return bool(np.any(dg < tie_gap) or np.any(vg < tie_gap))


def logits(o_concat: np.ndarray, w_u: np.ndarray) -> np.ndarray:
    """LM-head stand-in: concatenated head outputs times W_u (float64)."""
    return np.asarray(o_concat, dtype=np.float64) @ np.asarray(w_u, dtype=np.float64)
