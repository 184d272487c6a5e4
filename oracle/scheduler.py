"""Admit scheduler with a link ring and an HBM ring (plain Python).  Test infrastructure only.

Source: VeriCache review, §Runtime Algorithm Deep Dive ("Resource model", the Admit listing and
its line-by-line notes, "Execution loop").  The runtime looks W iterations ahead and keeps two
reserve rings: T[i], host-link time reserved for full-cache reloads landing in window i (the
link is serial, so T[i] <= T_iter), and B[i], full caches occupying HBM in window i (B[i] within
the HBM left after weights and resident caches).  A request's reload lasts
l_r = KV_full / (BW * T_iter) iterations and occupies S_r = max(1, ceil(l_r)) windows ending at
its verify.  Admit tries the verify slot d at the ideal draft length x first, then x+1, x-1,
x+2, x-2, ..., each clamped to [S_r, W-1], and reserves the first span [d - S_r + 1, d] that
fits both rings; if none fits the request waits.

Readings (the page does not spell these out):
* a reload's link time is spread evenly over its span: KV_full / (BW * S_r) per window;
* its whole KV_full is counted in HBM for every window of the span;
* "x +/- 1" is taken in the order written: x+1 before x-1;
* a reload longer than the window (S_r > W - 1) can never be admitted.
Windows are relative to the current iteration; advance() slides them by one, and a reservation
ends after its verify iteration.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple


class AdmitScheduler:
    def __init__(self, window: int, draft_len: int, t_iter: float, link_bw: float, hbm_budget: float):
        self.W, self.x = window, draft_len
        self.t_iter, self.bw, self.budget = t_iter, link_bw, hbm_budget
        self.now = 0
        self.T = [0.0] * window   # BW ring: link seconds reserved per window
        self.B = [0.0] * window   # HBM ring: bytes reserved per window
        self.res: Dict[int, Tuple[int, int]] = {}  # request -> (verify iteration, S_r)

    def candidates(self, S: int) -> List[int]:
        lo, hi = S, self.W - 1
        anchor = min(max(self.x, lo), hi)
        out = [anchor]
        for k in range(1, hi - lo + 1):
            out += [anchor + k, anchor - k]
        return [d for d in out if lo <= d <= hi]

    def admit(self, r: int, kv_full: float) -> Optional[int]:
        """The verify iteration reserved for r, or None (r waits)."""
        if r in self.res:
            raise ValueError("request already holds a reservation")
        ell = kv_full / (self.bw * self.t_iter)
        S = max(1, math.ceil(ell))
        if S > self.W - 1:
            return None
        per_window = kv_full / (self.bw * S)
        for d in self.candidates(S):
            span = range(d - S + 1, d + 1)
            link_ok = all(self.T[i] + per_window <= self.t_iter for i in span)
            hbm_ok = all(self.B[i] + kv_full <= self.budget for i in span)
            if link_ok and hbm_ok:
                for i in span:
                    self.T[i] += per_window
                    self.B[i] += kv_full
                self.res[r] = (self.now + d, S)
                return self.now + d
        return None

    def advance(self):
        self.res = {r: v for r, v in self.res.items() if v[0] > self.now}
        self.T = self.T[1:] + [0.0]
        self.B = self.B[1:] + [0.0]
        self.now += 1

    def due(self):
        """(requests whose reload starts now, requests that verify now), ascending ids."""
        reload = sorted(r for r, (d, S) in self.res.items() if d - S + 1 == self.now)
        verify = sorted(r for r, (d, S) in self.res.items() if d == self.now)
        return reload, verify
