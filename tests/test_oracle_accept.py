"""Pins of the oracle's argmax and greedy accept (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle.accept as acc
from oracle import workload
from vcsynth import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.json")


def test_golden_accept_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        assert acc.accept(c["draft"], c["verify"]) == (c["accept_len"], c["next"]), c["why"]


def test_planted_mismatch_positions():
    rng = np.random.default_rng(5)
    for x in (1, 5, 32, 40):
        base = rng.integers(0, 4096, size=x)
        assert acc.accept(base, base) == (x, -1)
        assert acc.accept(base, np.append(base, 77)) == (x, 77)
        for j in range(x):
            v = base.copy()
            v[j] = (v[j] + 1) % 4096
            v[j + 1:] = rng.integers(0, 4096, size=x - j - 1)  # anything after j is irrelevant
            assert acc.accept(base, v) == (j, int(v[j]))


def test_accept_rejects_bad_lengths():
    with pytest.raises(ValueError):
        acc.accept([1, 2, 3], [1])


def test_short_verifier_ends_the_block():
    """A verifier with fewer rows than drafted slots: only its rows are compared (hand cases)."""
    assert acc.accept_block([5, 7, 9, 11], [5, 7]) == (2, -1)      # both compared slots agree
    assert acc.accept_block([5, 7, 9, 11], [5, 6]) == (1, 6)       # mismatch inside the rows
    assert acc.accept_block([5, 7, 9, 11], []) == (0, -1)          # no verifier row at all
    assert acc.accept_block([5, 7, 9, 11], [4]) == (0, 4)
    # with x or x + 1 rows it is the plain rule
    assert acc.accept_block([5, 7], [5, 7, 3]) == (2, 3)
    assert acc.accept_block([5, 7], [5, 8]) == (1, 8)


def test_argmax_ties_and_gap():
    z = np.array([[0.0, 3.0, 3.0, 1.0], [5.0, -1.0, 4.5, 4.9], [2.0, 2.0, 2.0, 2.0]])
    t, gap = acc.argmax_gap(z)
    assert t.tolist() == [1, 0, 0]
    np.testing.assert_allclose(gap, [0.0, 0.1, 0.0], atol=1e-15)


def test_flags():
    # accept length 2 depends on rows 0..2; a near-tie at row 3 does not matter
    dg = np.array([1.0, 1.0, 1.0, 1e-5])
    vg = np.array([1.0, 1.0, 1.0, 1.0])
    assert not acc.accept_flagged(2, 4, dg, vg)
    assert acc.accept_flagged(3, 4, dg, vg)
    assert acc.accept_flagged(4, 4, dg, vg)


def test_logits_is_concat_times_wu():
    o = np.arange(6.0).reshape(1, 6)
    w = np.eye(6)[:, ::-1]
    assert acc.logits(o, w).tolist() == [[5.0, 4.0, 3.0, 2.0, 1.0, 0.0]]


def _keep_all(cfg):
    for r in cfg.reqs:
        r.comp, r.recent, r.top = configs.COMP_DROP, r.ctx_len, 0
    return cfg


def test_keep_all_draft_equals_verify_so_all_accepted():
    """Lossless compression makes the drafter and the verifier identical: a = x."""
    cfg = _keep_all(configs.scaled(configs.get("C1"), n=200))
    res = workload.round_instance(cfg, 0, 0)
    # same keys, same values: equal up to the summation order of the matrix products
    np.testing.assert_allclose(res.draft_o, res.verify_o, rtol=0, atol=1e-13)
    assert np.array_equal(res.draft_tok, res.verify_tok)
    assert res.accept_len == cfg.reqs[0].x and res.next_tok == -1


def test_lattice_kivi_draft_equals_verify():
    """Quantisation that is exact on its inputs also gives draft == verify (checked on lattice
    keys/values fed straight to the attention functions)."""
    from oracle import attention as att
    from oracle import compress as cmp
    rng = np.random.default_rng(3)
    n, d, x, G = 64, 64, 4, 2
    codes = rng.integers(0, 4, size=(n, d))
    codes[0::32] = 0
    codes[1::32] = 3
    codes[:, 0::32] = 0
    codes[:, 1::32] = 3
    kc = -0.375 + 0.25 * codes
    vc = -0.375 + 0.25 * codes[::-1]
    kq = cmp.dequantize_keys(*cmp.quantize_keys(kc, 2))
    vq = cmp.dequantize_values(*cmp.quantize_values(vc, 2))
    q = rng.normal(size=(x, G, d))
    kb, vb = rng.normal(size=(x, d)), rng.normal(size=(x, d))
    ver = att.verify_unit(q, kc, vc, kb, vb)
    assert np.array_equal(kq, kc) and np.array_equal(vq, vc)
    for i in range(x):
        np.testing.assert_allclose(att.draft_unit(q[i], kq, vq, kb, vb, i), ver[i], rtol=0, atol=1e-13)


def test_tiny_round_runs_and_is_consistent():
    cfg = configs.get("C1")
    res = workload.round_instance(cfg, 0, 0)
    x = cfg.reqs[0].x
    assert res.verify_o.shape == (x, cfg.Hq, cfg.d) and res.draft_o.shape == (x, cfg.Hq, cfg.d)
    a, nxt = acc.accept(res.draft_tok, res.verify_tok)
    assert (a, nxt) == (res.accept_len, res.next_tok)
    # dropping 3/4 of the context changes the output, but not wildly
    assert 0 < np.abs(res.draft_o - res.verify_o).max() < 1.0
