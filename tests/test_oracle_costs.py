"""Pins of the byte accounting against the pages' worked numbers."""
import json
import os

import pytest

from oracle import costs

W = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))


def test_kv_size_llama8b_100k():
    k = W["kv_size"]
    b = costs.kv_bytes(k["n"], k["L"], k["h"], k["d"], k["b"])
    assert b == 13_107_200_000
    assert abs(b / 1e9 - k["approx_gb"]) < 0.15


def test_eq3_worked_examples():
    m = W["eq3_mistral"]
    assert costs.iteration_hbm_bytes(m["M"], m["B"], m["kv_full"], m["c"], m["x"]) == pytest.approx(m["hbm_gb"])
    link = costs.iteration_link_bytes(m["B"], m["kv_full"], m["x"])
    assert link == pytest.approx(m["link_gb"])
    assert costs.transfer_seconds(link, m["link_gbps"]) * 1e3 == pytest.approx(m["t_xfer_ms_approx"], abs=0.5)
    q = W["eq3_qwen"]
    assert costs.iteration_hbm_bytes(q["M"], q["B"], q["kv_full"], q["c"], q["x"]) == pytest.approx(q["hbm_gb"])


def test_swap_transfer_time():
    s = W["swap_transfer"]
    assert costs.transfer_seconds(s["gb"], s["gbps"]) * 1e3 == pytest.approx(s["ms"])


def _t(w):
    return costs.iteration_time(w["M"], w["B"], w["kv_full"], w["c"], w["x"], w["bw_hbm_gbps"], w["bw_inter_gbps"])


def test_eq3_iteration_time_mistral():
    """T_gpu, T_xfer and the binding term of the Mistral-24B worked example (GB and GB/s)."""
    w = W["eq3_mistral_time"]
    t_gpu, t_xfer, t_iter = _t(w)
    assert t_gpu * 1e3 == pytest.approx(w["t_gpu_ms_approx"], abs=0.6)
    assert t_xfer * 1e3 == pytest.approx(w["t_xfer_ms_approx"], abs=0.5)
    assert t_iter == t_gpu and w["bound"] == "hbm"
    assert costs.effective_tokens(w["gamma"], w["x"]) == pytest.approx(w["eta_approx"], abs=0.005)
    assert costs.effective_tokens(w["gamma"], w["x"]) / t_iter == pytest.approx(w["tok_s_per_request_approx"], rel=0.02)
    assert costs.batch_tokens_per_second(w["B"], w["gamma"], w["x"], t_iter) == pytest.approx(w["tok_s_batch_approx"], rel=0.02)


def test_eq3_iteration_time_qwen():
    w = W["eq3_qwen_time"]
    t_gpu, t_xfer, t_iter = _t(w)
    assert t_gpu * 1e3 == pytest.approx(w["t_gpu_ms_approx"], abs=0.6)
    assert t_iter == t_gpu
    assert costs.effective_tokens(w["gamma"], w["x"]) / t_iter == pytest.approx(w["tok_s_per_request_approx"], rel=0.02)
    assert costs.batch_tokens_per_second(w["B"], w["gamma"], w["x"], t_iter) == pytest.approx(w["tok_s_batch_approx"], rel=0.02)


def test_eta_limits():
    """gamma = 0 leaves one token per iteration; gamma = 1 approaches 2 as x grows."""
    assert costs.effective_tokens(0.0, 25) == 1.0
    assert costs.effective_tokens(1.0, 1) == 1.5
    assert costs.effective_tokens(1.0, 10**9) == pytest.approx(2.0)


@pytest.mark.parametrize("M,B,kv,x,bh,bi", [(0.0, 8, 4.3, 32, 8000.0, 57.0), (48.0, 6, 5.0, 25, 1600.0, 64.0),
                                            (1.0, 1, 10.0, 30, 50.0, 1.0)])
def test_crossover_balances_eq3(M, B, kv, x, bh, bi):
    """At c* the two terms of Eq. (3) are equal; above it HBM binds, below it the link does."""
    cs = costs.crossover_compression(M, B, kv, x, bh, bi)
    t_gpu, t_xfer, _ = costs.iteration_time(M, B, kv, cs, x, bh, bi)
    assert t_gpu == pytest.approx(t_xfer, rel=1e-12)
    hi = costs.iteration_time(M, B, kv, cs + 0.01, x, bh, bi)
    lo = costs.iteration_time(M, B, kv, cs - 0.01, x, bh, bi)
    assert hi[0] > hi[1] and lo[0] < lo[1]


def test_crossover_typical_values():
    """The page's typical values (rho = 50, M/(B*KV_full) = 0.1, x = 30): solving Eq. (3) gives
    c* = 49/30 - 0.1, above 1, so every compression ratio leaves the link binding there."""
    cs = costs.crossover_compression(M=1.0, B=1, kv_full=10.0, x=30, bw_hbm=50.0, bw_inter=1.0)
    assert cs == pytest.approx(49 / 30 - 0.1)
    assert cs > 1.0
