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
