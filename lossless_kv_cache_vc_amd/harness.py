"""Device-side synthetic workload and one draft–verify round through the C ABI.

Inputs are drawn on the GPU by the seeded generator (``vcsynth``), packed into paged pools,
compressed by the library's own kernels, and run through draft attention (x single-query steps
over the compressed cache), verify attention (x causal rows over the full cache), the LM-head
stand-in and the greedy accept — the per-request cycle of the VeriCache review
(§Draft–Verify Pipeline).  PyTorch only allocates memory and provides the stream.
"""
from __future__ import annotations

import weakref
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from vcsynth import configs as C
from vcsynth import gpu as sg
from vcsynth import rng
from vcsynth.configs import NPOS, XMAX

from . import vc

BF16 = torch.bfloat16

# Guard regions around the tensors the kernels write (pools, outputs, workspaces, kept lists,
# logits, tokens) when VC_CANARY=1: each such tensor is a view into a larger buffer whose first and
# last CANARY_BYTES hold CANARY_BYTE, and check_canaries() reports any guard byte that changed (a
# write past either end).  Off by default; the tests turn it on.
CANARY_BYTES = 64 * 1024
CANARY_BYTE = 0xA5
_GUARDED: "weakref.WeakSet" = None


def _canary_on() -> bool:
    import os
    return os.environ.get("VC_CANARY") == "1"


def round16(x: int) -> int:
    return (x + 15) // 16 * 16


def _pages(n: int) -> int:
    return (n + 15) // 16


@dataclass
class Timing:
    ms: Dict[str, float] = field(default_factory=dict)


class Workload:
    """All device tensors of one configuration plus the launch lists of a round."""

    def __init__(self, cfg: C.Config, device: str = "cuda:0", build_compressed: bool = True,
                 keep_dense_scores: bool = False, spare_tokens: int = 0):
        """spare_tokens: growth room per request in every pool (page-table width, blocks handed
        out by the library's page allocator, kept-list width) for committing accepted rows."""
        self.cfg = cfg
        self._canary = _canary_on()
        self._guards = []
        if self._canary:
            global _GUARDED
            if _GUARDED is None:
                _GUARDED = weakref.WeakSet()
            _GUARDED.add(self)
        self.spare_pages = (spare_tokens + 15) // 16 + (1 if spare_tokens else 0)
        self.spare_tokens = spare_tokens
        self._grow = {}
        self.dev = torch.device(device)
        B, L, Hq, Hkv, d = cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.d
        self.xmax = round16(max(r.x for r in cfg.reqs))
        assert self.xmax <= XMAX
        self.shape = vc.shape(L, Hq, Hkv, d, self.xmax)
        seed = cfg.seed
        dev = self.dev
        with torch.cuda.device(dev):
            xm, P = self.xmax, self.xmax // 16
            self.q = torch.empty((B, L, xm, Hq, d), dtype=BF16, device=dev)
            sg.fill_normal_bf16(self.q, [L * XMAX * Hq * d, XMAX * Hq * d, Hq * d, d, 1], 0, seed,
                                rng.STREAM_Q)
            bs = [L * XMAX * Hkv * d, XMAX * Hkv * d, d, 16 * Hkv * d]
            self.blk_k = torch.empty((B, L, Hkv, P, 16, d), dtype=BF16, device=dev)
            sg.fill_normal_bf16(self.blk_k, bs + [Hkv * d, 1], 0, seed, rng.STREAM_KBLK)
            self.blk_v = torch.empty((B, L, Hkv, P, d, 16), dtype=BF16, device=dev)
            sg.fill_normal_bf16(self.blk_v, bs + [1, Hkv * d], 0, seed, rng.STREAM_VBLK)
            self.w_u = torch.empty((cfg.wu_width, cfg.vocab), dtype=BF16, device=dev)
            sg.fill_normal_bf16(self.w_u, [cfg.vocab, 1], 0, seed, rng.STREAM_WU, sigma=cfg.wu_sigma)

            self.lens = [r.ctx_len for r in cfg.reqs]
            self.comp_lens = [r.kept for r in cfg.reqs]
            self.full = self._bf16_pool(self.lens, salt=0, name="full")
            self._fill_full()

            self.out_v = self._out((B, L, xm, Hq, d), torch.float32, zero=True)
            self.out_d = self._out((B, L, xm, Hq, d), torch.float32, zero=True)
            self.drop_pool: Optional[vc.PagedPool] = None
            self.kivi_pool: Optional[vc.PagedPool] = None
            self.kept: Optional[torch.Tensor] = None
            if build_compressed:
                self._build_compressed(keep_dense_scores)
            self.workspace = self._workspace()

    # ---------------------------------------------------------------- guarded allocations
    def _out(self, shape, dtype, zero: bool = False) -> torch.Tensor:
        """A tensor the kernels write: inside guard regions when canaries are on."""
        if not self._canary:
            return (torch.zeros if zero else torch.empty)(shape, dtype=dtype, device=self.dev)
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        G = CANARY_BYTES
        buf = torch.empty(n + 2 * G, dtype=torch.uint8, device=self.dev)
        buf[:G].fill_(CANARY_BYTE)
        buf[G + n:].fill_(CANARY_BYTE)
        t = buf[G:G + n].view(dtype).view(shape)
        if zero:
            t.zero_()
        self._guards.append((buf, n))
        return t

    def check_canaries(self):
        """Raise AssertionError if a guard byte around a written tensor changed."""
        G = CANARY_BYTES
        for i, (buf, n) in enumerate(self._guards):
            lo, hi = buf[:G], buf[G + n:]
            if not (bool((lo == CANARY_BYTE).all()) and bool((hi == CANARY_BYTE).all())):
                bad_lo = int((lo != CANARY_BYTE).sum())
                bad_hi = int((hi != CANARY_BYTE).sum())
                raise AssertionError(f"guard bytes changed around written tensor {i} ({n} bytes): "
                                     f"{bad_lo} before it, {bad_hi} after it")

    # ---------------------------------------------------------------- pools
    def _tables(self, lens: List[int], salt: int, name: str):
        """Page tables and block count of a pool, with the growth room of spare_tokens: spare
        blocks after the initial ones, owned by a library page allocator (resident kind)."""
        cfg = self.cfg
        if not self.spare_pages:
            return C.page_tables(cfg.seed, lens, salt=salt)
        npages = max((n + 15) // 16 for n in lens)
        pt, nblk = C.page_tables(cfg.seed, lens, salt=salt, max_pages=npages + self.spare_pages)
        spare = len(lens) * self.spare_pages
        self._grow[name] = (pt, vc.PageAllocator(spare, spare), nblk)
        return pt, nblk + spare

    def _bf16_pool(self, lens: List[int], salt: int, name: str = "") -> vc.PagedPool:
        cfg = self.cfg
        pt, nblk = self._tables(lens, salt, name)
        shape = (cfg.L, nblk, cfg.Hkv, 16, cfg.d)
        k = self._out(shape, BF16)
        v = self._out(shape, BF16)
        return vc.PagedPool(16, torch.from_numpy(pt).to(self.dev), k, v, nblk)

    def _kivi_pool(self, lens: List[int], bits: int, salt: int, name: str = "") -> vc.PagedPool:
        cfg = self.cfg
        pt, nblk = self._tables(lens, salt, name)
        d, L, Hkv = cfg.d, cfg.L, cfg.Hkv
        k = self._out((L, nblk, Hkv, 16 * d * bits // 8), torch.uint8)
        v = self._out((L, nblk, Hkv, 16 * d * bits // 8), torch.uint8)
        ksz = self._out((L, nblk, Hkv, 2, d), torch.int16)
        vsz = self._out((L, nblk, Hkv, d // 32, 2, 16), torch.int16)
        return vc.PagedPool(bits, torch.from_numpy(pt).to(self.dev), k, v, nblk, ksz, vsz)

    @staticmethod
    def _row(pool: vc.PagedPool, r: int) -> vc.PagedPool:
        return Workload._rows(pool, r, r + 1)

    @staticmethod
    def _rows(pool: vc.PagedPool, r0: int, r1: int) -> vc.PagedPool:
        """The pool seen through page-table rows r0 .. r1 - 1 (they become rows 0 ..)."""
        return vc.PagedPool(pool.bits, pool.page_table[r0:r1], pool.k, pool.v, pool.num_blocks,
                            pool.k_sz, pool.v_sz)

    @staticmethod
    def _chunks(n: int):
        """Request ranges of at most vc.MAX_BATCH for the cache-building and commit calls."""
        return [(r0, min(n, r0 + vc.MAX_BATCH)) for r0 in range(0, n, vc.MAX_BATCH)]

    def _compress(self, lens, src: vc.PagedPool, kept, dst: vc.PagedPool, from_lens=None):
        """vc_compress / vc_compress_tail over the batch, in request ranges the calls accept."""
        stride = kept.shape[-1] if kept is not None else 0
        for r0, r1 in self._chunks(len(lens)):
            if not any(lens[r0:r1]):
                continue
            kk = kept[r0:r1] if kept is not None else None
            if from_lens is None:
                vc.compress(self.shape, lens[r0:r1], self._rows(src, r0, r1), kk, stride,
                            self._rows(dst, r0, r1))
            else:
                vc.compress_tail(self.shape, from_lens[r0:r1], lens[r0:r1], self._rows(src, r0, r1), kk,
                                 stride, self._rows(dst, r0, r1))

    def _fill_full(self):
        cfg = self.cfg
        Hkv, d, L = cfg.Hkv, cfg.d, cfg.L
        for r, n in enumerate(self.lens):
            if n == 0:
                continue
            src = torch.empty((1, Hkv, n, d), dtype=BF16, device=self.dev)
            row = self._row(self.full, r)
            for l in range(L):
                base = ((r * L + l) * Hkv) * NPOS * d
                for which, stream in ((0, rng.STREAM_KCTX), (1, rng.STREAM_VCTX)):
                    sg.fill_normal_bf16(src, [0, NPOS * d, d, 1], base, cfg.seed, stream)
                    vc.pack_bf16(self.shape, [n], l, src, n, row, which)
            del src

    def comp_len(self, r: int) -> int:
        return self.comp_lens[r]

    def drafts(self, r: int) -> bool:
        req = self.cfg.reqs[r]
        return req.kind != C.KIND_VERIFY

    def _build_compressed(self, keep_scores: bool):
        cfg = self.cfg
        B, L, Hkv = cfg.B, cfg.L, cfg.Hkv
        reqs = cfg.reqs
        drop_lens = [r.kept if (self.drafts(i) and r.comp in (C.COMP_DROP, C.COMP_DROP_KIVI4)) else 0
                     for i, r in enumerate(reqs)]
        kivi_lens = [r.kept if (self.drafts(i) and r.comp in (C.COMP_KIVI2, C.COMP_DROP_KIVI4)) else 0
                     for i, r in enumerate(reqs)]
        nmax = max(self.lens)
        if any(drop_lens):
            scores = torch.empty((B, L, Hkv, nmax), dtype=torch.int32, device=self.dev)
            sg.fill_u32(scores, [L * Hkv * NPOS, Hkv * NPOS, NPOS, 1], 0, cfg.seed, rng.STREAM_SCORE)
            kmax = max(drop_lens)
            self.kept = self._out((B, L, Hkv, kmax + self.spare_tokens), torch.int32)
            sel_lens = [n if k else 0 for n, k in zip(self.lens, drop_lens)]
            for r0, r1 in self._chunks(B):
                vc.select_kept(self.shape, sel_lens[r0:r1], [r.recent for r in reqs[r0:r1]],
                               [r.top for r in reqs[r0:r1]], scores[r0:r1], nmax, self.kept[r0:r1],
                               self.kept.shape[-1])
            if keep_scores:
                self.scores = scores
            else:
                del scores
        bf16_drop = [k if reqs[i].comp == C.COMP_DROP else 0 for i, k in enumerate(drop_lens)]
        if any(bf16_drop):
            self.drop_pool = self._bf16_pool(bf16_drop, salt=1, name="drop")
            self._compress(bf16_drop, self.full, self.kept, self.drop_pool)
        if any(kivi_lens):
            bits = {C.COMP_KIVI2: 2, C.COMP_DROP_KIVI4: 4}
            kinds = {reqs[i].comp for i, k in enumerate(kivi_lens) if k}
            assert len(kinds) == 1, "one KIVI bit width per workload"
            b = bits[kinds.pop()]
            self.kivi_pool = self._kivi_pool(kivi_lens, b, salt=2, name="kivi")
            with_kept = [k if reqs[i].comp == C.COMP_DROP_KIVI4 else 0 for i, k in enumerate(kivi_lens)]
            plain = [k if reqs[i].comp == C.COMP_KIVI2 else 0 for i, k in enumerate(kivi_lens)]
            if any(with_kept):
                self._compress(with_kept, self.full, self.kept, self.kivi_pool)
            if any(plain):
                self._compress(plain, self.full, None, self.kivi_pool)

    def draft_pool_of(self, r: int) -> vc.PagedPool:
        comp = self.cfg.reqs[r].comp
        return self.drop_pool if comp == C.COMP_DROP else self.kivi_pool

    # ---------------------------------------------------------------- launch lists
    def verify_reqs(self) -> List[vc.Req]:
        return [vc.Req(r, 0, n, r, 0, self.cfg.reqs[r].x, vc.VC_VERIFY)
                for r, n in enumerate(self.lens) if self.cfg.reqs[r].kind in (None, C.KIND_VERIFY)]

    def draft_reqs(self, step: int) -> List[vc.Req]:
        return [vc.Req(r, 0, self.comp_len(r), r, step, 1, vc.VC_DRAFT)
                for r in range(self.cfg.B) if step < self.cfg.reqs[r].x]

    def mixed_reqs(self) -> List[vc.Req]:
        """Ragged batch: pools 0 = full, 1 = bf16 drop, 2 = KIVI."""
        out = []
        for r, req in enumerate(self.cfg.reqs):
            if req.kind == C.KIND_DRAFT:
                pool = 1 if req.comp == C.COMP_DROP else 2
                out.append(vc.Req(r, pool, self.comp_lens[r], r, req.step, 1, vc.VC_DRAFT))
            else:
                out.append(vc.Req(r, 0, self.lens[r], r, 0, req.x, vc.VC_VERIFY))
        return out

    def mixed_pools(self) -> List[vc.PagedPool]:
        dummy = self.full
        return [self.full, self.drop_pool or dummy, self.kivi_pool or dummy]

    def _workspace(self) -> Optional[torch.Tensor]:
        need = 0
        if self.cfg.mixed:
            need = vc.attn_workspace_size(self.shape, self.mixed_reqs())
        else:
            need = vc.attn_workspace_size(self.shape, self.verify_reqs())
            if self.drop_pool is not None or self.kivi_pool is not None:
                for i in range(self.xmax):
                    rq = self.draft_reqs(i)
                    if rq:
                        need = max(need, vc.attn_workspace_size(self.shape, rq))
        if need == 0:
            return None
        return self._out((need // 4 + 1,), torch.float32)

    # ---------------------------------------------------------------- passes
    def run_verify(self, split_pages: int = 0, out: Optional[torch.Tensor] = None):
        vc.verify_attn(self.shape, self.verify_reqs(), self.q, self.blk_k, self.blk_v, self.full,
                       self.out_v if out is None else out, self.workspace_for(split_pages, "v"), split_pages)

    def run_draft(self, step: int, split_pages: int = 0, out: Optional[torch.Tensor] = None):
        rq = self.draft_reqs(step)
        if not rq:
            return
        pool = self.drop_pool if self.drop_pool is not None else self.kivi_pool
        vc.draft_attn(self.shape, rq, self.q, self.blk_k, self.blk_v, pool,
                      self.out_d if out is None else out, self.workspace_for(split_pages, "d", step),
                      split_pages)

    def run_mixed(self, split_pages: int = 0, out: Optional[torch.Tensor] = None):
        vc.attn_mixed(self.shape, self.mixed_reqs(), self.q, self.blk_k, self.blk_v, self.mixed_pools(),
                      self.out_v if out is None else out, self.workspace_for(split_pages, "m"), split_pages)

    def workspace_for(self, split_pages: int, which: str, step: int = 0):
        if split_pages == 0:
            return self.workspace
        rq = {"v": self.verify_reqs, "m": self.mixed_reqs}.get(which)
        reqs = rq() if rq else self.draft_reqs(step)
        need = vc.attn_workspace_size(self.shape, reqs, split_pages)
        if need == 0:
            return None
        key = ("ws", split_pages, which, step)
        cache = getattr(self, "_ws_cache", {})
        t = cache.get(key)
        if t is None or t.numel() * 4 < need:
            t = self._out((need // 4 + 1,), torch.float32)
            cache[key] = t
            self._ws_cache = cache
        return t

    # ---------------------------------------------------------------- commit / rollback
    def _extend(self, name: str, pool: vc.PagedPool, r: int, old: int, new: int):
        pt, alloc, base = self._grow[name]
        row = np.full(pt.shape[1], -1, dtype=np.int32)
        p_old = (old + 15) // 16
        alloc.extend_row(vc.PAGE_RESIDENT, row, old, new)      # ids of the spare range
        p_new = (new + 15) // 16
        if p_new > p_old:
            pt[r, p_old:p_new] = row[p_old:p_new] + base
            pool.page_table[r, p_old:p_new] = torch.from_numpy(pt[r, p_old:p_new].copy()).to(self.dev)

    def commit(self, counts: List[int]):
        """Append block rows [0, counts[r]) of request r (the K/V of the last accepted token and
        of the accepted drafted tokens) to its full cache at positions lens[r] .., and to its
        drafting cache: kept (token drop: new tokens are always kept), gathered or re-quantised
        from the full cache by the tail rebuild.  Rows from counts[r] on are rolled back, i.e. not
        committed.  Needs spare_tokens room."""
        cfg = self.cfg
        if not self.spare_pages:
            raise ValueError("commit needs a workload built with spare_tokens > 0")
        commits = []
        for r, c in enumerate(counts):
            if c <= 0:
                continue
            if c > cfg.reqs[r].x:
                raise ValueError("cannot commit more rows than were drafted")
            n, k = self.lens[r], self.comp_lens[r]
            self._extend("full", self.full, r, n, n + c)
            if self.drafts(r):
                comp = cfg.reqs[r].comp
                name, pool = ("drop", self.drop_pool) if comp == C.COMP_DROP else ("kivi", self.kivi_pool)
                self._extend(name, pool, r, k, k + c)
            commits.append((r, n, c, r, k))
        if not commits:
            return
        kept = self.kept
        dropped = lambda r: self.drafts(r) and cfg.reqs[r].comp in (C.COMP_DROP, C.COMP_DROP_KIVI4)
        with_kept = [c for c in commits if dropped(c[0])]
        without = [c for c in commits if not dropped(c[0])]
        step = vc.MAX_BATCH
        for i in range(0, len(with_kept), step):   # token drop: committed positions join the kept lists
            vc.commit_rows(self.shape, with_kept[i:i + step], self.blk_k, self.blk_v, self.full, kept,
                           kept.shape[-1])
        for i in range(0, len(without), step):
            vc.commit_rows(self.shape, without[i:i + step], self.blk_k, self.blk_v, self.full)
        for name, pool, comps in (("drop", self.drop_pool, (C.COMP_DROP,)),
                                  ("kivi", self.kivi_pool, (C.COMP_KIVI2, C.COMP_DROP_KIVI4))):
            if pool is None:
                continue
            for with_kept in (True, False):
                frm, to = [], []
                for r in range(cfg.B):
                    req = cfg.reqs[r]
                    uses = self.drafts(r) and req.comp in comps and \
                        (req.comp in (C.COMP_DROP, C.COMP_DROP_KIVI4)) == with_kept
                    c = counts[r] if uses else 0
                    frm.append(self.comp_lens[r] if uses else 0)
                    to.append(self.comp_lens[r] + c if uses else 0)
                if any(t > f for f, t in zip(frm, to)):
                    self._compress(to, self.full, kept if with_kept else None, pool, from_lens=frm)
        for r, n, c, _, k in commits:
            self.lens[r] = n + c
            if self.drafts(r):
                self.comp_lens[r] = k + c
        self.workspace = self._workspace()

    def logits(self):
        """LM-head stand-in for both passes (z_v, z_d: [B*L*xmax][vocab] fp32)."""
        cfg = self.cfg
        B, L, xm, V = cfg.B, cfg.L, self.xmax, cfg.vocab
        width = cfg.Hq * cfg.d
        rows = B * L * xm
        if not hasattr(self, "z_v"):
            self.z_v = self._out((rows, V), torch.float32)
            self.z_d = self._out((rows, V), torch.float32)
            xs = torch.tensor([cfg.reqs[r].x for r in range(B) for _ in range(L)], dtype=torch.int32)
            self.x_dev = xs.to(self.dev)
            self.tok_d = self._out((B * L, xm), torch.int32)
            self.tok_v = self._out((B * L, xm), torch.int32)
            self.acc_len = self._out((B * L,), torch.int32)
            self.next_tok = self._out((B * L,), torch.int32)
        vc.logits(rows, width, V, self.out_v, width, self.w_u, self.z_v)
        vc.logits(rows, width, V, self.out_d, width, self.w_u, self.z_d)

    def accept(self, temperature: float = 0.0):
        """Greedy accept (temperature 0), or drafted tokens sampled from the drafter's logits and
        the rejection-sampling accept (seeded uniforms, generated once).  Needs logits()."""
        cfg = self.cfg
        B, L, xm, V = cfg.B, cfg.L, self.xmax, cfg.vocab
        if temperature <= 0:
            vc.accept(B * L, xm, xm, V, self.x_dev, self.x_dev, self.z_d, self.z_v, self.tok_d, self.tok_v,
                      self.acc_len, self.next_tok)
            return
        if not hasattr(self, "u_draft"):
            idx = np.arange(B * L * xm, dtype=np.int64)
            self.u_draft = torch.from_numpy(rng.uniform01(cfg.seed, rng.STREAM_UDRAFT, idx)).to(self.dev)
            self.u_acc = torch.from_numpy(rng.uniform01(cfg.seed, rng.STREAM_UACC, idx)).to(self.dev)
            self.u_res = torch.from_numpy(rng.uniform01(cfg.seed, rng.STREAM_URES,
                                                        np.arange(B * L * (xm + 1), dtype=np.int64))).to(self.dev)
        vc.sample_tokens(B * L * xm, V, temperature, self.z_d, self.u_draft, self.tok_d)
        vc.accept_sampled(B * L, xm, xm, V, temperature, self.x_dev, self.x_dev, self.z_d, self.z_v, self.tok_d,
                          self.u_acc, self.u_res, self.acc_len, self.next_tok)

    def logits_and_accept(self, temperature: float = 0.0):
        self.logits()
        self.accept(temperature)

    def run_round(self):
        """x draft steps, the verify pass, logits of both, accept."""
        for i in range(max(r.x for r in self.cfg.reqs)):
            self.run_draft(i)
        self.run_verify()
        self.logits_and_accept()

    # ---------------------------------------------------------------- staging the full cache
    def full_to_host(self):
        """Copy the full pool's K and V into exact-size pinned host buffers (the host tier the full
        cache is reloaded from).  Returns the two buffers; keep them alive while staging."""
        from .pinned import PinnedBuffer
        bufs = []
        for t in (self.full.k, self.full.v):
            b = PinnedBuffer(t.numel() * t.element_size())
            b.tensor(t.dtype, t.shape).copy_(t)
            bufs.append(b)
        torch.cuda.synchronize(self.dev)
        return bufs

    def stage_full(self, bufs, side_stream, event, layers: Optional[int] = None):
        """Enqueue the reload of the full pool from `bufs` (full_to_host) on `side_stream` with
        vc_stage_kv, one copy per layer slice of K and of V, and record `event` after the last one.
        layers: reload only layer slices [0, layers).  Returns the bytes enqueued."""
        L = self.cfg.L if layers is None else layers
        if event is not None:
            event.record(side_stream)   # torch creates the HIP event on its first record
        total = 0
        for t, b in zip((self.full.k, self.full.v), bufs):
            per = t[0].numel() * t.element_size()
            host = b.tensor(t.dtype, t.shape)
            for l in range(L):
                vc.stage_kv(t[l], host[l], per, side_stream, event)
                total += per
        return total

    # ---------------------------------------------------------------- algorithmic bytes
    def verify_bytes(self) -> int:
        """Bytes the verify pass must move: context K/V, drafted-block K/V, Q, O, page tables."""
        cfg = self.cfg
        tot = 0
        for r in self.verify_reqs():
            x = r.rows
            tot += cfg.L * cfg.Hkv * (r.ctx_len * cfg.d * 2 * 2 + x * cfg.d * 2 * 2)
            tot += cfg.L * x * cfg.Hq * cfg.d * (2 + 4)
            tot += _pages(r.ctx_len) * 4
        return tot

    def draft_bytes(self, step: int) -> int:
        """Bytes one draft step must move: the compressed cache, visible drafted rows, q, o."""
        cfg = self.cfg
        tot = 0
        for r in self.draft_reqs(step):
            tot += cfg.L * cfg.Hkv * self.comp_token_bytes(r.slot) * r.ctx_len
            tot += cfg.L * cfg.Hkv * (step + 1) * cfg.d * 2 * 2
            tot += cfg.L * cfg.Hq * cfg.d * (2 + 4)
            tot += _pages(r.ctx_len) * 4
        return tot

    def comp_token_bytes(self, r: int) -> float:
        """Bytes per stored token and kv head of request r's drafting cache."""
        d = self.cfg.d
        req = self.cfg.reqs[r]
        if req.comp == C.COMP_DROP:
            return 2 * d * 2
        b = req.bits
        # K and V codes, value (scale, zero) per 32 channels, key (scale, zero) per 32 tokens
        return 2 * d * b / 8 + (d // 32) * 4 + d * 4 / 32

    def mixed_bytes(self) -> int:
        cfg = self.cfg
        tot = 0
        for r in self.mixed_reqs():
            if r.kind == vc.VC_VERIFY:
                tot += cfg.L * cfg.Hkv * (r.ctx_len + r.rows) * cfg.d * 4
                tot += cfg.L * r.rows * cfg.Hq * cfg.d * 6
            else:
                tot += int(cfg.L * cfg.Hkv * (self.comp_token_bytes(r.slot) * r.ctx_len +
                                              (r.q0 + 1) * cfg.d * 4))
                tot += cfg.L * cfg.Hq * cfg.d * 6
            tot += _pages(r.ctx_len) * 4
        return tot


def check_all_canaries():
    """Check the guard regions of every live workload built with canaries (VC_CANARY=1)."""
    if _GUARDED is None:
        return
    torch.cuda.synchronize()
    for wl in list(_GUARDED):
        wl.check_canaries()
