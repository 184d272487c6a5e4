"""The parity gate's error model, checked on the CPU against a simulation of the rounding.

The attention kernels round each softmax weight before the value product and divide by row sums
of the unrounded weights.  Weights are exponentials relative to a running maximum:
* bf16 weights (verify, bf16 draft): the running maximum moves whenever a row's maximum grows,
  so the key that sets it has weight exactly 1 and every other weight is rounded to 8 bits;
* fp16 weights (KIVI draft): the running maximum may lag the row's maximum by up to 8 (log2
  units), and every weight is rounded to 11 bits.
Simulated here in float64 on rows of N(0, sigma^2) scores over 40 to 32K keys: at the workloads'
score scale (sigma = 1) every error sits within ``gate(spread)``, the contract included; on
peaked rows (sigma = 3, a few keys carry the row) within the model's uncapped bound.  On long
rows the gate stays within a small factor of the errors seen (it is not vacuous).
"""
import numpy as np
import pytest

from gpu_helpers import SIGMA_W_BF16, SIGMA_W_KIVI, TOL_CONTRACT, gate
import oracle.attention as att


def round_bits(x, mant):
    """Round float32 values to ``mant`` significant bits, to nearest even (bf16: 8, fp16: 11;
    normal range only, which these weights stay in)."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    sh = 24 - mant
    half = (1 << (sh - 1)) - 1
    b = ((b + half + ((b >> sh) & 1)) >> sh) << sh
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def simulate(n, sigma, rows, rng, mant, lagmax, d=64):
    s = rng.normal(scale=sigma, size=(rows, n))
    v = rng.normal(size=(n, d))
    lag = rng.uniform(0.0, lagmax, size=(rows, 1)) if lagmax > 0 else 0.0
    e = np.exp2(s * np.log2(np.e) - (s.max(axis=1, keepdims=True) * np.log2(np.e) - lag))
    l = e.sum(axis=1, keepdims=True)
    err = np.abs((round_bits(e, mant) - e) @ v / l)
    wn = e / l
    return err, np.sqrt((wn * wn) @ (v * v))


@pytest.mark.parametrize("n", [40, 137, 330, 1000, 32768])
def test_bf16_weights_within_the_gate_at_the_workload_scale(n):
    rng = np.random.default_rng(7 + n)
    rows = 40 if n > 1000 else 20000
    err, spr = simulate(n, 1.0, rows, rng, mant=8, lagmax=0.0)
    g = gate(spr)
    assert np.all(err <= g), float((err / g).max())
    if n >= 1000:
        assert float((err / g).max()) > 0.03     # not vacuous
        assert float(np.median(g)) < TOL_CONTRACT / 2  # typical rows: well inside the contract


@pytest.mark.parametrize("mant,lagmax,sigma_w", [(8, 0.0, SIGMA_W_BF16), (11, 8.0, SIGMA_W_KIVI)])
def test_peaked_rows_within_the_uncapped_model(mant, lagmax, sigma_w):
    rng = np.random.default_rng(3)
    err, spr = simulate(137, 3.0, 20000, rng, mant=mant, lagmax=lagmax)
    assert np.all(err <= 12.0 * sigma_w * spr + 1e-4)


@pytest.mark.parametrize("n", [40, 137, 4096])
def test_fp16_weights_within_the_kivi_gate(n):
    rng = np.random.default_rng(11 + n)
    err, spr = simulate(n, 1.0, 20000 if n < 4096 else 400, rng, mant=11, lagmax=8.0)
    assert np.all(err <= gate(spr, kivi=True))


def test_a_lagging_maximum_would_break_the_contract_with_bf16_weights():
    """Why the bf16 paths move the running maximum eagerly: with 8 units of headroom the key that
    dominates a short row keeps a rounded weight, and rows of 40 keys then exceed the contract."""
    rng = np.random.default_rng(11 + 40)
    err, _ = simulate(40, 1.0, 200000, rng, mant=8, lagmax=8.0)
    assert float(err.max()) > TOL_CONTRACT
    rng = np.random.default_rng(11 + 40)
    err, _ = simulate(40, 1.0, 200000, rng, mant=8, lagmax=0.0)
    assert float(err.max()) < 0.6 * TOL_CONTRACT


def test_rounding_helper_matches_torch():
    import torch
    x = np.random.default_rng(5).normal(size=10000).astype(np.float32) * 100
    assert np.array_equal(round_bits(x, 8), torch.from_numpy(x).bfloat16().double().numpy())
    assert np.array_equal(round_bits(x, 11), torch.from_numpy(x).half().double().numpy())


def test_spread_of_the_oracle_matches_the_simulation_formula():
    """The spread the simulation uses is the one the oracle returns for the same weights."""
    rng = np.random.default_rng(3)
    d, n = 16, 50
    q, k, v = rng.normal(size=(4, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    _, spr = att.attention(q, k, v, spread=True)
    s = q @ k.T / np.sqrt(d)
    w = np.exp(s - s.max(axis=1, keepdims=True)); w /= w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(spr, np.sqrt((w * w) @ (v * v)), rtol=1e-12)
