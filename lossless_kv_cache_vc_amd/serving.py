"""One-GPU draft/verify serving loop: full caches reloaded from pinned host memory, staggered by
the library's Admit scheduler, against lock-step reloads and a resident full cache.

VeriCache review, §KV Swap Scheduling (lock-step vs staggered) and §Runtime Algorithm Deep Dive
("Execution loop"): at each iteration, start the reloads whose reserved span begins now, run the
drafting requests' next step, run the verifies scheduled now (each waits for its reload), and
re-admit every request that verified.  Lock-step instead reloads every request's full cache at
once (serialised on the link), verifies them all, then drafts x iterations.

Each request's full cache is one contiguous bf16 pool (identity page table), so a reload is two
pinned-host-to-HBM copies (vc_stage_kv) on a side stream; a verify waits on its reload's event.
Staged caches land in a small set of device slots: a slot is reused only after the verify that
read it has run (the side stream waits on that verify's event).  Drafting uses the workload's
compressed cache and drafted block.  This is an experiment driver; the attention, the staging and
the scheduling are the library's.

    python -m lossless_kv_cache_vc_amd.serving --n 8192 --iters 400
"""
from __future__ import annotations

import argparse
import json
import math
import time
from typing import Dict, List, Optional

import torch

from vcsynth import configs as C

from . import vc
from .harness import Workload


class ServeLoop:
    def __init__(self, cfg: C.Config, staged: bool = True):
        self.cfg = cfg
        self.wl = Workload(cfg)
        wl = self.wl
        dev = wl.dev
        B, L, Hkv, d = cfg.B, cfg.L, cfg.Hkv, cfg.d
        self.x = cfg.reqs[0].x
        self.n = [r.ctx_len for r in cfg.reqs]
        self.npages = [(n + 15) // 16 for n in self.n]
        # contiguous per-request full caches gathered from the workload's shared pool
        self.full_k, self.full_v, self.tables = [], [], []
        for r in range(B):
            ids = wl.full.page_table[r, :self.npages[r]].long()
            self.full_k.append(wl.full.k.index_select(1, ids).contiguous())
            self.full_v.append(wl.full.v.index_select(1, ids).contiguous())
            self.tables.append(torch.arange(self.npages[r], dtype=torch.int32, device=dev).view(1, -1))
        self.kv_bytes = [self.full_k[r].numel() * 2 * 2 for r in range(B)]
        self.staged = staged
        if staged:
            self.host_k = [t.cpu().pin_memory() for t in self.full_k]
            self.host_v = [t.cpu().pin_memory() for t in self.full_v]
        wl.full = None  # the shared pool is no longer read
        torch.cuda.empty_cache()
        # one workspace for every launch of the loop: split planning depends on how many
        # requests a launch holds, so take the largest need over draft launches of 1..B requests
        # and a single-request verify
        need = max(vc.attn_workspace_size(wl.shape, [vc.Req(r, 0, self.n[r], 0, 0, self.x, vc.VC_VERIFY)])
                   for r in range(B))
        for k in range(1, B + 1):
            need = max(need, vc.attn_workspace_size(
                wl.shape, [vc.Req(r, 0, wl.comp_len(r), r, 0, 1, vc.VC_DRAFT) for r in range(k)]))
        self.ws = torch.empty(need // 4 + 1, dtype=torch.float32, device=dev) if need else None
        self.main = torch.cuda.current_stream()
        self.side = torch.cuda.Stream()

    # ------------------------------------------------------------------ pieces of an iteration
    def pool_of(self, r: int, k: torch.Tensor, v: torch.Tensor) -> vc.PagedPool:
        return vc.PagedPool(16, self.tables[r], k, v, self.npages[r])

    def draft(self, steps: Dict[int, int]):
        """One draft launch for the requests in `steps` (request -> draft step)."""
        wl = self.wl
        reqs = [vc.Req(r, 0, wl.comp_len(r), r, i, 1, vc.VC_DRAFT) for r, i in sorted(steps.items())]
        if reqs:
            pool = wl.drop_pool if wl.drop_pool is not None else wl.kivi_pool
            vc.draft_attn(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pool, wl.out_d, self.ws)

    def verify(self, r: int, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None):
        wl = self.wl
        req = [vc.Req(r, 0, self.n[r], 0, 0, self.x, vc.VC_VERIFY)]
        vc.verify_attn(wl.shape, req, wl.q, wl.blk_k, wl.blk_v, self.pool_of(r, k, v),
                       wl.out_v if out is None else out, self.ws)

    def stage(self, r: int, k: torch.Tensor, v: torch.Tensor, after: Optional[torch.cuda.Event]) -> torch.cuda.Event:
        """Reload request r's full cache into (k, v) on the side stream; returns its event."""
        if after is not None:
            self.side.wait_event(after)
        ev = torch.cuda.Event()
        ev.record(self.side)  # the event object exists before the library records it
        vc.stage_kv(k, self.host_k[r], k.numel() * k.element_size(), self.side, None)
        vc.stage_kv(v, self.host_v[r], v.numel() * v.element_size(), self.side, ev)
        return ev

    # ------------------------------------------------------------------ modes
    def run_resident(self, iters: int) -> dict:
        """Full caches stay in HBM: every request verifies every x iterations, verifies spread
        evenly over the cycle; no reloads."""
        B, x = self.cfg.B, self.x
        offset = {r: (r * x) // B for r in range(B)}
        verifies = 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for it in range(iters):
            due = [r for r in range(B) if (it + 1 - offset[r]) % x == 0 and it + 1 >= offset[r]]
            self.draft({r: (it - offset[r]) % x for r in range(B) if r not in due})
            for r in due:
                self.verify(r, self.full_k[r], self.full_v[r])
                verifies += 1
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"mode": "resident", "iters": iters, "wall_s": wall, "verifies": verifies}

    def run_lockstep(self, iters: int) -> dict:
        """Every x iterations all requests reload (serialised on the link) and then verify."""
        B, x = self.cfg.B, self.x
        slots = [(torch.empty_like(self.full_k[r]), torch.empty_like(self.full_v[r])) for r in range(B)]
        verifies, it = 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while it < iters:
            for i in range(min(x, iters - it)):
                self.draft({r: i for r in range(B)})
                it += 1
            evs = [self.stage(r, *slots[r], None) for r in range(B)]
            for r in range(B):
                self.main.wait_event(evs[r])
                self.verify(r, *slots[r])
                verifies += 1
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"mode": "lockstep", "iters": iters, "wall_s": wall, "verifies": verifies,
                "peak_full_caches_in_hbm": B}

    def run_staggered(self, iters: int, t_iter: float, link_bw: float, slots_n: int = 2,
                      window: int = 0) -> dict:
        """The library's Admit scheduler places each request's reload and verify."""
        B, x = self.cfg.B, self.x
        kv = max(self.kv_bytes)
        ell = kv / (link_bw * t_iter)
        W = window or max(2 * x, int(math.ceil(ell)) * (B + 1) + 2)
        sched = vc.Scheduler(W, x, t_iter, link_bw, slots_n * kv)
        slots = [(torch.empty_like(self.full_k[0]), torch.empty_like(self.full_v[0])) for _ in range(slots_n)]
        free = list(range(slots_n))
        slot_of: Dict[int, int] = {}
        staged_ev: Dict[int, torch.cuda.Event] = {}
        slot_done: List[Optional[torch.cuda.Event]] = [None] * slots_n
        admitted_at: Dict[int, int] = {}
        waiting = list(range(B))
        verifies, peak = 0, 0

        def try_admit():
            for r in list(waiting):
                if sched.admit(r, self.kv_bytes[r]) is not None:
                    waiting.remove(r)
                    admitted_at[r] = sched.now

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        try_admit()
        for it in range(iters):
            reload, verify = sched.due()
            for r in reload:
                s = free.pop()
                slot_of[r] = s
                staged_ev[r] = self.stage(r, *slots[s], slot_done[s])
            peak = max(peak, slots_n - len(free))
            drafting = {r: (sched.now - a) % x for r, a in admitted_at.items() if r not in verify}
            self.draft(drafting)
            for r in verify:
                s = slot_of.pop(r)
                self.main.wait_event(staged_ev.pop(r))
                self.verify(r, *slots[s])
                done = torch.cuda.Event()
                done.record(self.main)
                slot_done[s] = done
                free.append(s)
                verifies += 1
                admitted_at.pop(r)
                waiting.append(r)
            sched.advance()
            try_admit()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"mode": "staggered", "iters": iters, "wall_s": wall, "verifies": verifies, "window": W,
                "reload_windows": int(max(1, math.ceil(ell))), "peak_full_caches_in_hbm": peak}

    # ------------------------------------------------------------------ calibration
    def measure(self, reps: int = 5):
        """(seconds per draft-only iteration, link bytes per second)."""
        B, x = self.cfg.B, self.x
        for _ in range(2):
            self.draft({r: 0 for r in range(B)})
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps * 4):
            self.draft({r: i % x for r in range(B)})
        torch.cuda.synchronize()
        t_iter = (time.perf_counter() - t0) / (reps * 4)
        bw = None
        if self.staged:
            k, v = torch.empty_like(self.full_k[0]), torch.empty_like(self.full_v[0])
            self.stage(0, k, v, None).synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                self.stage(0, k, v, None).synchronize()
            bw = self.kv_bytes[0] * reps / (time.perf_counter() - t0)
        return t_iter, bw


def main(argv=None):
    ap = argparse.ArgumentParser(description="staggered vs lock-step full-cache reloads on one GPU")
    ap.add_argument("--config", default="C2")
    ap.add_argument("--n", type=int, default=8192, help="context tokens per request")
    ap.add_argument("--iters", type=int, default=400)
    args = ap.parse_args(argv)
    cfg = C.scaled(C.get(args.config), n=args.n)
    loop = ServeLoop(cfg)
    t_iter, bw = loop.measure()
    B, x = cfg.B, loop.x
    tokens = lambda res: res["verifies"] * x  # drafted tokens verified (every drafted token kept)
    out = {"workload": f"{cfg.name}, n = {args.n}, B = {B}, x = {x}", "kv_full_bytes": loop.kv_bytes[0],
           "t_draft_iter_s": t_iter, "link_bytes_per_s": bw, "rho": None, "modes": []}
    for res in (loop.run_resident(args.iters), loop.run_staggered(args.iters, t_iter, bw),
                loop.run_lockstep(args.iters)):
        res["iter_ms"] = res["wall_s"] / res["iters"] * 1e3
        res["verified_tokens_per_s"] = tokens(res) / res["wall_s"]
        out["modes"].append(res)
        print(json.dumps(res), flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
