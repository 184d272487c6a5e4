"""Pins of the oracle's compressed cache (token drop and KIVI-style quantisation)."""
import itertools

import numpy as np
import pytest

import oracle.compress as cmp
from oracle.numerics import fp16_to_f64

RNG = np.random.default_rng(99)


def brute_kept(scores, n, R, m):
    """Enumerate every m-subset of the older positions; keep the lexicographically best
    (highest score multiset, then lowest positions)."""
    older = n - R
    best = None
    for sub in itertools.combinations(range(older), m):
        key = (sorted([-int(scores[p]) for p in sub]), list(sub))
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(list(best[1]) + list(range(older, n)))


@pytest.mark.parametrize("n,R,m", [(9, 2, 3), (10, 0, 4), (8, 8, 0), (7, 3, 4)])
def test_kept_positions_brute_force(n, R, m):
    for trial in range(5):
        scores = RNG.integers(0, 4, size=n).astype(np.uint32)  # many ties on purpose
        got = cmp.kept_positions(scores, n, R, m)
        assert got.tolist() == brute_kept(scores, n, R, m)


def test_kept_positions_invariants_large():
    n, R, m = 32768, 128, 8192
    scores = RNG.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    kept = cmp.kept_positions(scores, n, R, m)
    assert len(kept) == R + m
    assert np.all(np.diff(kept) > 0)
    assert set(range(n - R, n)) <= set(kept.tolist())
    older = kept[kept < n - R]
    dropped = np.setdiff1d(np.arange(n - R), older)
    assert scores[older].min() >= scores[dropped].max()


def test_kept_positions_ties_prefer_lower_positions():
    scores = np.array([5, 7, 7, 7, 7, 1], dtype=np.uint32)
    assert cmp.kept_positions(scores, 6, 1, 2).tolist() == [1, 2, 5]


def test_kept_positions_clamps():
    assert cmp.kept_positions(np.zeros(5, np.uint32), 5, 10, 10).tolist() == [0, 1, 2, 3, 4]


def test_key_quantisation_hand_example():
    # one channel, 4 tokens [-1, -0.5, 0, 0.5] with 2 bits: min -1, max 0.5,
    # scale = 1.5 / 3 = 0.5, zero = -1, codes 0..3, exact reconstruction
    k = np.array([[-1.0], [-0.5], [0.0], [0.5]])
    codes, s, z = cmp.quantize_keys(k, 2)
    assert codes[:, 0].tolist() == [0, 1, 2, 3]
    assert fp16_to_f64(s).tolist() == [[0.5]] and fp16_to_f64(z).tolist() == [[-1.0]]
    assert np.array_equal(cmp.dequantize_keys(codes, s, z), k)


def test_quantisation_groups_follow_kivi_convention():
    # keys: groups run along tokens per channel; values: groups run along channels per token
    T, d = 64, 64
    k = RNG.normal(size=(T, d))
    codes, s, z = cmp.quantize_keys(k, 2)
    assert s.shape == (2, d)
    for g in range(2):
        blk = k[g * 32:(g + 1) * 32]
        np.testing.assert_array_equal(z[g], blk.min(0).astype(np.float16))
    v = RNG.normal(size=(T, d))
    vc, vs, vz = cmp.quantize_values(v, 4)
    assert vs.shape == (T, 2)
    np.testing.assert_array_equal(vz[:, 1], v[:, 32:64].min(1).astype(np.float16))


@pytest.mark.parametrize("bits", [2, 4])
def test_dequantisation_error_bound(bits):
    T, d = 100, 128  # includes a short last key group (100 = 3*32 + 4)
    L = (1 << bits) - 1
    for x, fn, deq, axis in [(RNG.normal(size=(T, d)), cmp.quantize_keys, cmp.dequantize_keys, 0),
                             (RNG.normal(size=(T, d)), cmp.quantize_values, cmp.dequantize_values, 1)]:
        codes, s, z = fn(x, bits)
        assert codes.max() <= L
        xh = deq(codes, s, z)
        if axis == 0:
            grp = np.arange(T) // 32
            sf, zf = fp16_to_f64(s)[grp], fp16_to_f64(z)[grp]
            mn = np.stack([x[g * 32:(g + 1) * 32].min(0) for g in range(4)])[grp]
            mx = np.stack([x[g * 32:(g + 1) * 32].max(0) for g in range(4)])[grp]
        else:
            ch = np.arange(d) // 32
            sf, zf = fp16_to_f64(s)[:, ch], fp16_to_f64(z)[:, ch]
            xg = x.reshape(T, d // 32, 32)
            mn, mx = xg.min(2)[:, ch], xg.max(2)[:, ch]
        # rounding to the nearest level costs s/2; fp16 rounding of scale and zero moves the
        # covered range by at most L*|s - (mx-mn)/L| + |z - mn|
        bound = sf / 2 + L * np.abs(sf - (mx - mn) / L) + np.abs(zf - mn) + 1e-12
        assert np.all(np.abs(x - xh) <= bound)
        assert np.abs(x - xh).max() <= (sf.max() / 2) * 1.01


@pytest.mark.parametrize("bits", [2, 4])
def test_lattice_inputs_reconstruct_exactly(bits):
    # values on the lattice z + code * s with s = 1/4, z = -3/8 (exact in fp16 and bf16) and
    # codes 0 and 2^b - 1 present in every quantisation group: quantisation is lossless
    L = (1 << bits) - 1
    s, z = 0.25, -0.375
    T, d = 64, 64
    kcodes = RNG.integers(0, L + 1, size=(T, d))
    kcodes[0::32, :] = 0          # key groups run along tokens
    kcodes[1::32, :] = L
    vcodes = RNG.integers(0, L + 1, size=(T, d))
    vcodes[:, 0::32] = 0          # value groups run along channels
    vcodes[:, 1::32] = L
    for codes, fn, deq in [(kcodes, cmp.quantize_keys, cmp.dequantize_keys),
                           (vcodes, cmp.quantize_values, cmp.dequantize_values)]:
        x = z + codes * s
        c, sc, zz = fn(x, bits)
        assert np.array_equal(c, codes)
        assert np.all(fp16_to_f64(sc) == s) and np.all(fp16_to_f64(zz) == z)
        assert np.array_equal(deq(c, sc, zz), x)


def test_constant_group_has_zero_scale():
    k = np.full((32, 4), 1.25)
    codes, s, z = cmp.quantize_keys(k, 2)
    assert np.all(fp16_to_f64(s) == 0) and np.all(codes == 0)
    assert np.array_equal(cmp.dequantize_keys(codes, s, z), k)
