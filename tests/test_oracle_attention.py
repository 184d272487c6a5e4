"""Pins of the oracle's attention (draft and verify passes) on the CPU.

What fixes the answer, other than the oracle itself: a library routine (torch's
scaled_dot_product_attention in float64), brute force with Python scalars, closed forms,
and invariants of softmax attention (row weights sum to 1, key-permutation invariance,
split-and-merge equals unsplit, causal prefix consistency, x = 1 verify equals a decode step).
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as att

RNG = np.random.default_rng(1234)


def brute_force(q, k, v):
    """Softmax attention with Python floats and explicit loops (tiny inputs only)."""
    rows, d = len(q), len(q[0])
    out = []
    for i in range(rows):
        s = [sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d) for j in range(len(k))]
        m = max(s)
        w = [math.exp(t - m) for t in s]
        tot = sum(w)
        out.append([sum(w[j] * v[j][c] for j in range(len(k))) / tot for c in range(d)])
    return np.array(out)


def test_brute_force_tiny():
    q = RNG.normal(size=(3, 4))
    k = RNG.normal(size=(5, 4))
    v = RNG.normal(size=(5, 4))
    np.testing.assert_allclose(att.attention(q, k, v), brute_force(q.tolist(), k.tolist(), v.tolist()),
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("G,x,n,d", [(4, 8, 200, 64), (8, 5, 97, 128), (1, 3, 33, 32)])
def test_verify_matches_torch_sdpa(G, x, n, d):
    q = RNG.normal(size=(x, G, d))
    kc, vc = RNG.normal(size=(n, d)), RNG.normal(size=(n, d))
    kb, vb = RNG.normal(size=(x, d)), RNG.normal(size=(x, d))
    got = att.verify_unit(q, kc, vc, kb, vb)
    keys = torch.from_numpy(np.concatenate([kc, kb]))
    vals = torch.from_numpy(np.concatenate([vc, vb]))
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [G][x][d]
    mask = torch.ones(x, n + x, dtype=torch.bool)
    mask[:, n:] = torch.tril(torch.ones(x, x, dtype=torch.bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, keys.expand(G, -1, -1), vals.expand(G, -1, -1), attn_mask=mask)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_draft_matches_torch_sdpa():
    G, d, k, step = 4, 128, 300, 6
    q = RNG.normal(size=(G, d))
    kc, vc = RNG.normal(size=(k, d)), RNG.normal(size=(k, d))
    kb, vb = RNG.normal(size=(10, d)), RNG.normal(size=(10, d))
    got = att.draft_unit(q, kc, vc, kb, vb, step)
    keys = torch.from_numpy(np.concatenate([kc, kb[:step + 1]]))
    vals = torch.from_numpy(np.concatenate([vc, vb[:step + 1]]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], keys[None], vals[None])[0]
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_equal_keys_give_mean_of_values():
    d, n = 16, 50
    k = np.tile(RNG.normal(size=(1, d)), (n, 1))
    v = RNG.normal(size=(n, d))
    q = RNG.normal(size=(3, d))
    np.testing.assert_allclose(att.attention(q, k, v), np.tile(v.mean(0), (3, 1)), atol=1e-14)


def test_constant_values_give_that_value():
    d, n = 16, 40
    v = np.tile(RNG.normal(size=(1, d)), (n, 1))
    out = att.attention(RNG.normal(size=(2, d)), RNG.normal(size=(n, d)), v)
    np.testing.assert_allclose(out, np.tile(v[0], (2, 1)), atol=1e-14)


def test_dominant_key_selects_its_value():
    d, n = 32, 64
    k = RNG.normal(size=(n, d)) * 0.01
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k[17, 0] = 60.0 * math.sqrt(d)  # score 60 above the rest: weight of others < n e^-59
    v = RNG.normal(size=(n, d))
    np.testing.assert_allclose(att.attention(q, k, v)[0], v[17], atol=1e-20 + 1e-12)


def test_rows_are_probability_distributions():
    n, d = 37, 8
    q, k = RNG.normal(size=(5, d)), RNG.normal(size=(n, d))
    w = att.attention(q, k, np.eye(n))       # one-hot values expose the weights
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)


def test_key_permutation_invariance():
    n, d = 80, 32
    q, k, v = RNG.normal(size=(4, d)), RNG.normal(size=(n, d)), RNG.normal(size=(n, d))
    p = RNG.permutation(n)
    np.testing.assert_allclose(att.attention(q, k, v), att.attention(q, k[p], v[p]), atol=1e-14)


def test_split_and_merge_equals_unsplit():
    n, d = 300, 64
    q, k, v = RNG.normal(size=(6, d)), RNG.normal(size=(n, d)), RNG.normal(size=(n, d))
    full = att.attention(q, k, v)
    # each part's (max, sum, weighted sum), merged with log-sum-exp weights
    parts = []
    for lo, hi in [(0, 70), (70, 71), (71, 300)]:
        s = q @ k[lo:hi].T / math.sqrt(d)
        m = s.max(1, keepdims=True)
        w = np.exp(s - m)
        parts.append((m, w.sum(1, keepdims=True), w @ v[lo:hi]))
    M = np.max(np.concatenate([p[0] for p in parts], 1), 1, keepdims=True)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    np.testing.assert_allclose(num / den, full, rtol=1e-12, atol=1e-14)


def test_verify_row_is_attention_over_its_prefix():
    G, x, n, d = 2, 6, 50, 16
    q = RNG.normal(size=(x, G, d))
    kc, vc, kb, vb = (RNG.normal(size=s) for s in [(n, d), (n, d), (x, d), (x, d)])
    out = att.verify_unit(q, kc, vc, kb, vb)
    for i in range(x):
        keys = np.concatenate([kc, kb[:i + 1]])
        vals = np.concatenate([vc, vb[:i + 1]])
        np.testing.assert_allclose(out[i], att.attention(q[i], keys, vals), atol=1e-14)


def test_verify_x1_equals_decode_step():
    G, n, d = 4, 77, 32
    q = RNG.normal(size=(1, G, d))
    kc, vc, kb, vb = (RNG.normal(size=s) for s in [(n, d), (n, d), (1, d), (1, d)])
    v1 = att.verify_unit(q, kc, vc, kb, vb)[0]
    d0 = att.draft_unit(q[0], kc, vc, kb, vb, 0)  # keep-all "compressed" cache
    assert np.array_equal(v1, d0)


def test_gqa_group_one_is_mha():
    n, d, x = 40, 16, 3
    q = RNG.normal(size=(x, 1, d))
    kc, vc, kb, vb = (RNG.normal(size=s) for s in [(n, d), (n, d), (x, d), (x, d)])
    out = att.verify_unit(q, kc, vc, kb, vb)[:, 0]
    for i in range(x):
        keys = np.concatenate([kc, kb[:i + 1]])
        vals = np.concatenate([vc, vb[:i + 1]])
        np.testing.assert_allclose(out[i], brute_force(q[i].tolist(), keys.tolist(), vals.tolist())[0],
                                   atol=1e-13)
    assert [att.gqa_group(h, 4) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong scale or an exclusive causal mask in the oracle fails the library pin."""
    G, x, n, d = 2, 4, 30, 16
    q = RNG.normal(size=(x, G, d))
    kc, vc, kb, vb = (RNG.normal(size=s) for s in [(n, d), (n, d), (x, d), (x, d)])
    keys = torch.from_numpy(np.concatenate([kc, kb]))
    vals = torch.from_numpy(np.concatenate([vc, vb]))
    mask = torch.ones(x, n + x, dtype=torch.bool)
    mask[:, n:] = torch.tril(torch.ones(x, x, dtype=torch.bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), keys.expand(G, -1, -1), vals.expand(G, -1, -1),
        attn_mask=mask).permute(1, 0, 2).numpy()
    good = att.verify_unit(q, kc, vc, kb, vb)
    assert np.abs(good - ref).max() < 1e-12

    real = att.attention

    def wrong_scale(q_, k_, v_, visible=None):
        return real(q_ * math.sqrt(q_.shape[-1]) ** -1, k_, v_, visible)  # scale 1/d
    monkeypatch.setattr(att, "attention", wrong_scale)
    assert np.abs(att.verify_unit(q, kc, vc, kb, vb) - ref).max() > 1e-3
    monkeypatch.setattr(att, "attention", real)

    def exclusive_mask(q_, k_, v_, visible=None):
        vis = visible.copy()
        for r in range(vis.shape[0]):
            vis[r, n + r // G] = False  # drop the row's own drafted key
        return real(q_, k_, v_, vis)
    monkeypatch.setattr(att, "attention", exclusive_mask)
    assert np.abs(att.verify_unit(q, kc, vc, kb, vb) - ref).max() > 1e-3


def test_spread_closed_forms_and_unchanged_output():
    """The weight spread sqrt(sum_t (w_t v_tc)^2): |v| of a key that takes all the weight,
    |c| / sqrt(n) for equal weights over n keys with constant values c, a brute-force sum in
    general; asking for it leaves the output unchanged."""
    d, n = 8, 6
    q = np.zeros((1, d))
    k = RNG.normal(size=(n, d))
    v = np.full((n, d), -3.0)
    out, spr = att.attention(q, k, v, spread=True)           # q = 0: equal weights
    np.testing.assert_allclose(spr, np.full((1, d), 3.0 / np.sqrt(n)), rtol=1e-14)
    np.testing.assert_allclose(out, v[:1], rtol=1e-14)
    q = np.zeros((1, d)); q[0, 0] = 1e4                        # one key dominates
    k = np.zeros((n, d)); k[2, 0] = 1.0
    v = RNG.normal(size=(n, d))
    out, spr = att.attention(q, k, v, spread=True)
    np.testing.assert_allclose(spr[0], np.abs(v[2]), rtol=1e-12)
    q, k, v = RNG.normal(size=(3, d)), RNG.normal(size=(n, d)), RNG.normal(size=(n, d))
    vis = np.tril(np.ones((3, n), dtype=bool), k=3)
    out, spr = att.attention(q, k, v, vis, spread=True)
    assert np.array_equal(out, att.attention(q, k, v, vis))
    for i in range(3):
        s = np.where(vis[i], k @ q[i] / np.sqrt(d), -np.inf)
        w = np.exp(s - s.max()); w /= w.sum()
        want = [math.sqrt(sum((w[t] * v[t, c]) ** 2 for t in range(n))) for c in range(d)]
        np.testing.assert_allclose(spr[i], want, rtol=1e-12)
