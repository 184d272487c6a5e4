"""Pins of the Admit scheduler oracle (VeriCache review, §Runtime Algorithm Deep Dive and §KV Swap
Scheduling "Concrete numbers from the paper")."""
import json
import os

from oracle.scheduler import AdmitScheduler

W = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "scheduler_worked.json")))


def test_single_request_verifies_at_the_draft_length():
    s = AdmitScheduler(window=64, draft_len=30, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s.admit(0, 0.5) == 30            # l = 0.5: one window
    s2 = AdmitScheduler(window=64, draft_len=30, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s2.admit(0, 2.5) == 30           # l = 2.5: three windows, [28, 30]
    assert s2.T[27] == 0 and all(abs(s2.T[i] - 2.5 / 3) < 1e-15 for i in (28, 29, 30)) and s2.T[31] == 0
    assert s2.B[28:31] == [2.5] * 3


def test_clamps_of_the_anchor():
    s = AdmitScheduler(window=16, draft_len=30, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s.admit(0, 0.1) == 15            # x beyond the window: the last window
    s = AdmitScheduler(window=64, draft_len=2, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s.admit(0, 4.5) == 5             # S = 5 > x: the verify cannot come before S
    s = AdmitScheduler(window=8, draft_len=4, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s.admit(0, 7.5) is None          # S = 8 > W - 1: never fits


def test_serial_link_staggers_reloads():
    """Three reloads each filling the link for 3 windows: verifies at x, x+3, x-3."""
    s = AdmitScheduler(window=64, draft_len=30, t_iter=1.0, link_bw=1.0, hbm_budget=100.0)
    assert [s.admit(r, 3.0) for r in range(3)] == [30, 33, 27]
    assert max(s.T) <= 1.0


def test_hbm_budget_staggers_reloads():
    """A light link but room for one full cache at a time: spans may not overlap."""
    s = AdmitScheduler(window=64, draft_len=30, t_iter=1.0, link_bw=10.0, hbm_budget=5.0)
    assert [s.admit(r, 4.0) for r in range(3)] == [30, 31, 29]
    assert max(s.B) <= 5.0
    s = AdmitScheduler(window=64, draft_len=30, t_iter=1.0, link_bw=10.0, hbm_budget=3.0)
    assert s.admit(0, 4.0) is None          # larger than the whole budget: waits


def test_advance_and_due():
    s = AdmitScheduler(window=16, draft_len=4, t_iter=1.0, link_bw=1.0, hbm_budget=10.0)
    assert s.admit(7, 1.5) == 4             # S = 2: reload from iteration 3, verify at 4
    seen = []
    for _ in range(6):
        seen.append((s.now, s.due()))
        s.advance()
    assert seen[3] == (3, ([7], [])) and seen[4] == (4, ([], [7]))
    assert not s.res and s.T == [0.0] * 16  # the reservation ended after its verify
    assert s.admit(7, 1.5) == s.now + 4     # and the request can be admitted again


def test_concrete_swap_scenario_of_the_page():
    """Ten requests, 4 GB full caches reloaded in about 80 ms over the link, 35 ms iterations,
    x = 30: verifies spread one every 3 iterations and only one full cache is in HBM at a time;
    lock-step would serialise all ten reloads (about 800 ms, some 20 iteration windows)."""
    w = W["swap_scenario"]
    bw = w["kv_full_bytes"] / w["transfer_s"]
    s = AdmitScheduler(window=w["window"], draft_len=w["x"], t_iter=w["t_iter_s"], link_bw=bw,
                       hbm_budget=w["hbm_budget_bytes"])
    d = sorted(s.admit(r, w["kv_full_bytes"]) for r in range(w["B"]))
    assert all(b - a == w["verify_spacing"] for a, b in zip(d, d[1:]))
    assert max(s.B) == w["kv_full_bytes"] * w["max_full_caches_in_hbm"]
    lock_step_link = w["B"] * w["transfer_s"]
    assert abs(lock_step_link - w["lock_step_link_s"]) < 1e-12
    assert round(lock_step_link / w["t_iter_s"]) >= w["lock_step_windows_at_least"]
