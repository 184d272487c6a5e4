"""Pins of the rejection-sampling accept oracle (VeriCache review, §Implementation notes,
"Rejection sampling for non-greedy"): closed forms of the pieces, the control flow of a
block, and the property the page states -- the emitted token follows p_full exactly --
measured on tiny vocabularies with a deterministic grid over each uniform."""
import numpy as np
import pytest

from oracle import sampling as S


def test_probs_closed_form():
    p = S.probs(np.array([0.0, np.log(3.0)]), 1.0)
    assert p == pytest.approx([0.25, 0.75], rel=1e-15)
    p = S.probs(np.array([0.0, np.log(3.0)]), 0.5)   # 3^2 = 9
    assert p == pytest.approx([0.1, 0.9], rel=1e-14)
    with pytest.raises(ValueError):
        S.probs(np.zeros(3), 0.0)


def test_draw_intervals():
    w = np.ones(4)
    assert [S.draw(w, u)[0] for u in (0.1, 0.26, 0.49, 0.51, 0.99)] == [0, 1, 1, 2, 3]
    w = np.array([0.0, 2.0, 0.0, 1.0])     # [0, 2/3) -> 1, [2/3, 1) -> 3
    assert [S.draw(w, u)[0] for u in (1e-9, 0.6, 0.67, 0.999)] == [1, 1, 3, 3]
    k, margin = S.draw(np.ones(4), 0.5 + 1e-12)  # right at a boundary
    assert k == 2 and margin < S.NEAR


def _grid(n):
    return (np.arange(n) + 0.5) / n


def _emitted_distribution(zd, zv, T, n):
    """P(first emitted token = k) of one slot (x = 1, no bonus row), measured by running the
    oracle over a regular grid of each uniform: the draft draw, the keep test, the residual
    draw.  The three uniforms are independent, so the probabilities multiply."""
    V = zd.shape[-1]
    g = _grid(n)
    pt = np.bincount([S.draw(S.probs(zd, T), u)[0] for u in g], minlength=V) / n
    out = np.zeros(V)
    for t in range(V):
        if pt[t] == 0:
            continue
        kept = np.mean([S.accept_sampled(zd[None], zv[None], [t], T, [u], [0.5])[0] == 1 for u in g])
        out[t] += pt[t] * kept
        if kept < 1:
            # a uniform just below 1 always rejects a token the keep test can reject
            res = [S.accept_sampled(zd[None], zv[None], [t], T, [1 - 1e-15], [u]) for u in g]
            assert all(r[0] == 0 for r in res)
            out += pt[t] * (1 - kept) * np.bincount([r[1] for r in res], minlength=V) / n
    return out


@pytest.mark.parametrize("seed,V,T", [(1, 4, 1.0), (2, 5, 0.7), (3, 6, 0.3), (4, 3, 1.0)])
def test_emitted_token_follows_p_full(seed, V, T):
    rng = np.random.default_rng(seed)
    zd = rng.normal(0, 1.5, V)
    zv = rng.normal(0, 1.5, V)
    n = 4000
    got = _emitted_distribution(zd, zv, T, n)
    pf, pl = S.probs(zv, T), S.probs(zd, T)
    # each measured interval length is within 1/n of the true one (midpoint grid); a handful
    # of intervals enter each probability
    assert np.abs(got - pf).max() < 12.0 / n
    # and the drafter's own distribution is visibly different, so the check has teeth
    assert np.abs(pl - pf).max() > 0.05


def test_identical_caches_keep_every_slot():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 1, (4, 7))
    toks, _ = S.sample_tokens(z[:3], 0.8, [0.3, 0.6, 0.9])
    a, nxt, _ = S.accept_sampled(z[:3], z[:3], toks, 0.8, [0.999999] * 3, [0.5] * 4)
    assert (a, nxt) == (3, -1)
    a, nxt, _ = S.accept_sampled(z[:3], z, toks, 0.8, [0.999999] * 3, [0.5] * 4)
    assert a == 3 and nxt == S.draw(S.probs(z[3], 0.8), 0.5)[0]


def test_token_the_verifier_rules_out_is_rejected():
    """p_full(t) underflows to 0: the slot is rejected whatever u, and the replacement comes
    from where p_full exceeds p_lossy."""
    zd = np.array([[0.0, 0.0, 0.0, 0.0]])
    zv = np.array([[0.0, 1.0, -1e4, 2.0]])
    for u in (1e-6, 0.5, 0.999):
        a, nxt, _ = S.accept_sampled(zd, zv, [2], 1.0, [u], [u])
        pf, pl = S.probs(zv[0], 1.0), S.probs(zd[0], 1.0)
        assert a == 0 and pf[nxt] > pl[nxt]


def test_stops_at_first_rejection():
    zd = np.zeros((3, 4))
    zv = np.array([[0.0, 0.0, 0.0, 0.0], [0.0, -1e4, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    a, nxt, _ = S.accept_sampled(zd, zv, [1, 1, 1], 1.0, [0.5] * 3, [0.5] * 4)
    assert a == 1 and nxt in (0, 2, 3)


def test_low_temperature_matches_greedy():
    rng = np.random.default_rng(9)
    zd = rng.normal(0, 1, (5, 9))
    zv = zd.copy()
    zv[3] = rng.normal(0, 1, 9)
    toks, _ = S.sample_tokens(zd, 1e-3, rng.uniform(size=5))
    assert np.array_equal(toks, zd.argmax(-1))
    a, nxt, _ = S.accept_sampled(zd, zv, toks, 1e-3, rng.uniform(size=5), rng.uniform(size=6))
    if zd[3].argmax() != zv[3].argmax():
        assert (a, nxt) == (3, int(zv[3].argmax()))
