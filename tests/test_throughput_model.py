"""The throughput-model calculator against the oracle's Eq. (3) and acceptance model, and its
bench-fed mode on a synthetic bench line (no GPU)."""
import numpy as np
import pytest

from lossless_kv_cache_vc_amd import throughput as tm
from oracle import costs


def test_calculator_matches_oracle():
    rng = np.random.default_rng(7)
    for _ in range(200):
        M = float(rng.uniform(0, 100e9))
        B = int(rng.integers(1, 65))
        kv = float(rng.uniform(0.1e9, 70e9))
        c = float(rng.uniform(0.01, 1.0))
        x = int(rng.integers(1, 65))
        bh, bi = float(rng.uniform(1e12, 8e12)), float(rng.uniform(10e9, 500e9))
        got = tm.t_iter(M, B, kv, c, x, bh, bi)
        t_gpu, t_xfer, t_iter = costs.iteration_time(M, B, kv, c, x, bh, bi)
        assert got.hbm_bytes == pytest.approx(costs.iteration_hbm_bytes(M, B, kv, c, x), rel=1e-14)
        assert got.xfer_bytes == pytest.approx(costs.iteration_link_bytes(B, kv, x), rel=1e-14)
        assert (got.t_gpu, got.t_xfer, got.t_iter) == pytest.approx((t_gpu, t_xfer, t_iter), rel=1e-14)
        assert got.bound == ("hbm" if t_gpu >= t_xfer else "interconnect")
        assert tm.c_star(bh / bi, x, M / (B * kv)) == pytest.approx(
            costs.crossover_compression(M, B, kv, x, bh, bi), rel=1e-9, abs=1e-12)
        g = float(rng.uniform(0, 1))
        assert tm.eta(g, x) == pytest.approx(costs.effective_tokens(g, x), rel=1e-15)
        assert tm.tokens_per_s(B, tm.eta(g, x), t_iter) == pytest.approx(
            costs.batch_tokens_per_second(B, g, x, t_iter), rel=1e-14)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        tm.t_iter(0, 1, 1.0, 0.2, 0, 1.0, 1.0)


def _bench_line():
    # the shape of a bench.py line at the Llama-3.1-8B 32K workload (numbers made up)
    return {"config": {"workload": "synthetic", "batch": 8, "x": 32},
            "bytes": {"verify": 34.59e9, "draft_per_step_avg": 8.75e9},
            "breakdown_ms": {"draft_per_launch": 1.30, "verify": 5.94}}


def test_from_bench_round_bytes_and_identities():
    b = _bench_line()
    r = tm.from_bench(b, stage_gbps=57.0)
    B, x = 8, 32
    # x iterations of Eq. (3) with M = 0 carry exactly one round's bytes: x draft steps + one verify
    assert r["eq3_at_peak_hbm"]["hbm_bytes"] * x == pytest.approx(b["bytes"]["verify"] + x * b["bytes"]["draft_per_step_avg"])
    assert r["kv_full_GB"] == pytest.approx(34.59 / B)
    assert r["c"] == pytest.approx(8.75 / 34.59)
    # with M = 0, Eq. (3)'s HBM term at the measured kernel rates is the measured iteration
    assert r["t_gpu_at_measured_rates_s"] == pytest.approx(r["t_iter_measured_gpu_s"], rel=1e-12)
    assert r["t_iter_measured_gpu_s"] == pytest.approx((1.30 + 5.94 / x) * 1e-3)
    # one full KV per request every x iterations over a 57 GB/s link
    assert r["t_xfer_s"] == pytest.approx(34.59e9 / x / 57e9)
    assert r["bound_measured"] == "interconnect"
    assert r["rho_peak"] == pytest.approx(8000 / 57)


def test_from_bench_with_gamma():
    r = tm.from_bench(_bench_line(), stage_gbps=57.0, gamma=0.9)
    assert r["eta"] == pytest.approx(1 + 0.9 * 32 / 33)
    assert r["tokens_per_s_measured_gpu"] == pytest.approx(8 * r["eta"] / r["t_xfer_s"])
