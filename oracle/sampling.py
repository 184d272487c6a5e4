"""Rejection-sampling accept for temperature > 0 (float64).  Test infrastructure only.

Source: VeriCache review, §Implementation notes worth absorbing, "Rejection sampling for
non-greedy" (and §Background on speculative decoding): the drafter samples t_i from its own
distribution p_lossy; the verifier evaluates p_full(t_i) and keeps t_i with probability
min(1, p_full(t_i) / p_lossy(t_i)); at the first slot it does not keep, one token is drawn from
the residual distribution (p_full - p_lossy, negative parts removed, renormalised) and the block
ends there.  The emitted tokens then follow p_full exactly.

Readings (the page gives the rule in one sentence):
* p = softmax(z / T) over the vocabulary, computed in float64 from the fp32 logits, T > 0.
* Drawing from weights w (not necessarily normalised) with a uniform u in (0, 1): the smallest
  index k whose prefix sum w_0 + ... + w_k exceeds u * sum(w).  If rounding leaves no prefix
  above it, the last index with w_k > 0.
* The keep test for slot i is u_acc[i] * p_lossy(t_i) < p_full(t_i): the same event as
  u_acc[i] < p_full / p_lossy, with no division (a ratio of at least 1 always keeps).
* If every drafted slot is kept and the verifier gave an (x+1)-th row, the bonus token is drawn
  from p_full of that row with u_res[x]; with x rows only there is no next token (-1), as in the
  greedy accept.
* If the residual has no mass (p_full = p_lossy to the last bit) a rejection cannot occur in exact
  arithmetic; the draw then falls back to p_full.
* Every decision is compared with its threshold; a decision closer than a relative 1e-9 is
  flagged "near tie", since another float64 evaluation order may take the other side.
"""
from __future__ import annotations

import numpy as np

NEAR = 1e-9


def probs(z: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(z / T) in float64 over the last axis."""
    if not temperature > 0:
        raise ValueError("temperature must be > 0")
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp((z - m) / temperature)
    return e / e.sum(axis=-1, keepdims=True)


def draw(weights: np.ndarray, u: float):
    """(index, margin): inverse-CDF draw from non-negative `weights` with uniform u.

    margin is the distance of u*sum(w) to the nearest boundary of the chosen index's interval,
    relative to sum(w)."""
    w = np.asarray(weights, dtype=np.float64)
    total = w.sum()
    target = u * total
    cdf = np.cumsum(w)
    above = np.nonzero(cdf > target)[0]
    if len(above):
        k = int(above[0])
    else:
        k = int(np.nonzero(w > 0)[0][-1])
    lo = cdf[k - 1] if k > 0 else 0.0
    margin = min(abs(target - lo), abs(cdf[k] - target)) / total if total > 0 else 0.0
    return k, margin


def sample_tokens(z: np.ndarray, temperature: float, u: np.ndarray):
    """Draft-side sampling: one token per row of z [rows][V] with uniforms u [rows].
    Returns (tokens, near-tie flags)."""
    p = probs(z, temperature)
    toks, flags = [], []
    for r in range(p.shape[0]):
        k, margin = draw(p[r], float(u[r]))
        toks.append(k)
        flags.append(margin < NEAR)
    return np.array(toks, dtype=np.int64), np.array(flags)


def accept_sampled(z_draft: np.ndarray, z_verify: np.ndarray, draft_tok, temperature: float,
                   u_acc, u_res):
    """(accept length a, next token, flagged) for one drafted block.

    z_draft [x][V] are the drafter's logits for the x slots, z_verify [x or x+1][V] the
    verifier's; draft_tok [x] the drafted tokens; u_acc [x] and u_res [x+1] uniforms in (0, 1)."""
    x = len(draft_tok)
    xv = z_verify.shape[0]
    if xv not in (x, x + 1):
        raise ValueError("verifier must give x or x + 1 rows")
    pl = probs(z_draft, temperature)
    pf = probs(z_verify, temperature)
    flagged = False
    for i in range(x):
        t = int(draft_tok[i])
        lhs, rhs = float(u_acc[i]) * pl[i, t], pf[i, t]
        if abs(lhs - rhs) <= NEAR * max(lhs, rhs):
            flagged = True
        if lhs < rhs:
            continue
        resid = np.maximum(pf[i] - pl[i], 0.0)
        if resid.sum() == 0.0:
            resid = pf[i]
        k, margin = draw(resid, float(u_res[i]))
        return i, k, flagged or margin < NEAR
    if xv == x + 1:
        k, margin = draw(pf[x], float(u_res[x]))
        return x, k, flagged or margin < NEAR
    return x, -1, flagged
