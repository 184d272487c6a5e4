"""The five synthetic workloads: shapes, seeds, compression settings and per-request draws.

Everything here is data (sizes, seeds, which compression each request uses) plus draws from the
counter generator; no attention, compression or accept arithmetic lives here.

Logical index conventions (layout-independent; every tensor value is
``value(seed, stream, logical_index)``):

* Q        [B][L][XMAX][Hq][d]           stream 1
* K, V ctx [B][L][Hkv][NPOS][d]          streams 2, 3 (position-major per kv head)
* K, V blk [B][L][XMAX][Hkv][d]          streams 4, 5 (the drafted block's own K/V rows)
* W_u      [width][vocab]                stream 6
* score    [B][L][Hkv][NPOS]             stream 7 (uint32; larger = more important)
* draws    [B][16]                       stream 8 (ragged-batch lengths, kinds, steps, modes)
* pages    one draw per physical block   stream 9 (random page placement)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
from scipy.special import ndtri

from . import rng

XMAX = 64          # largest drafted block (query rows per request)
NPOS = 1 << 20     # logical position stride of the context tensors
BLOCK = 16         # tokens per KV page

# per-request compression of the drafting KV cache
COMP_DROP = "drop"            # keep recent R + top-m by score, bf16
COMP_KIVI2 = "kivi2"          # all tokens, 2-bit KIVI-style
COMP_DROP_KIVI4 = "drop+kivi4"  # drop as above, then 4-bit KIVI-style over the kept sequence

KIND_VERIFY = 0
KIND_DRAFT = 1


@dataclass
class Request:
    ctx_len: int                 # n_r
    x: int                       # drafted block length / verify rows
    comp: str                    # compression of this request's drafting cache
    recent: int = 0              # R (drop)
    top: int = 0                 # m (drop)
    kind: Optional[int] = None   # ragged batch only: KIND_VERIFY or KIND_DRAFT
    step: int = 0                # ragged batch draft step i_r

    @property
    def kept(self) -> int:
        """k_r: tokens in the drafting cache."""
        if self.comp == COMP_KIVI2:
            return self.ctx_len
        return min(self.ctx_len, self.recent + self.top)

    @property
    def bits(self) -> int:
        return {COMP_DROP: 16, COMP_KIVI2: 2, COMP_DROP_KIVI4: 4}[self.comp]


@dataclass
class Config:
    name: str
    cid: int
    L: int
    Hq: int
    Hkv: int
    d: int
    reqs: List[Request]
    wu_width: int
    vocab: int
    mixed: bool = False          # single ragged draft+verify launch
    staged: bool = False         # full KV staged from pinned host memory
    note: str = ""

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.cid

    @property
    def B(self) -> int:
        return len(self.reqs)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def wu_sigma(self) -> float:
        return 1.0 / math.sqrt(self.wu_width)

    def full_kv_bytes(self) -> int:
        """Bytes of bf16 K and V over every request's full context (2*n*L*h*d*2 per request)."""
        return sum(2 * r.ctx_len * self.L * self.Hkv * self.d * 2 for r in self.reqs)


def _drop_req(n, x, R, m):
    return Request(ctx_len=n, x=x, comp=COMP_DROP, recent=R, top=m)


def c1_tiny() -> Config:
    return Config("C1-tiny", 1, L=1, Hq=8, Hkv=2, d=64,
                  reqs=[_drop_req(1024, 8, 64, 192)], wu_width=512, vocab=1024,
                  note="1 request, n=1024, keep last 64 + 192 random, x=8")


def c2_llama8b_32k() -> Config:
    n = 32768
    return Config("C2-llama8b-32k", 2, L=32, Hq=32, Hkv=8, d=128,
                  reqs=[_drop_req(n, 32, 128, n // 4) for _ in range(8)],
                  wu_width=4096, vocab=4096,
                  note="Llama-3.1-8B attention shape, n=32768, B=8, x=32, 4x token drop")


def c3_llama8b_100k_kivi2() -> Config:
    n = 100000
    return Config("C3-llama8b-100k-kivi2", 3, L=32, Hq=32, Hkv=8, d=128,
                  reqs=[Request(ctx_len=n, x=32, comp=COMP_KIVI2) for _ in range(4)],
                  wu_width=4096, vocab=4096,
                  note="Llama-3.1-8B shape, n=100000, B=4, x=32, KIVI 2-bit")


def c4_qwen32b_128k() -> Config:
    n = 131072
    return Config("C4-qwen32b-128k", 4, L=64, Hq=64, Hkv=8, d=128,
                  reqs=[Request(ctx_len=n, x=40, comp=COMP_DROP_KIVI4, recent=128, top=n // 4)
                        for _ in range(2)],
                  wu_width=8192, vocab=4096, staged=True,
                  note="Qwen-32B-like shape, n=131072, B=2, x=40, 4x drop + KIVI 4-bit")


def c5_ragged(nreq: int = 64) -> Config:
    cid = 5
    seed = 0x5EED0000 + cid
    idx = np.arange(nreq, dtype=np.int64) * 16
    # context lengths: ln n ~ N(ln sqrt(4096*131072), (ln 32 / 4)^2), rounded, clipped
    mu = math.log(math.sqrt(4096.0 * 131072.0))
    sg = math.log(32.0) / 4.0
    z = ndtri(rng.uniform01(seed, rng.STREAM_DRAWS, idx + 0))
    n = np.clip(np.rint(np.exp(mu + sg * z)), 4096, 131072).astype(np.int64)
    # half of the requests draft: a seeded permutation picks them
    perm = np.argsort(rng.u32(seed, rng.STREAM_DRAWS, idx + 1), kind="stable")
    drafting = np.zeros(nreq, dtype=bool)
    drafting[perm[: nreq // 2]] = True
    step = (rng.u32(seed, rng.STREAM_DRAWS, idx + 2) % np.uint32(40)).astype(np.int64)
    mode = (rng.u32(seed, rng.STREAM_DRAWS, idx + 3) >> np.uint32(31)).astype(np.int64)
    xv = 8 + (rng.u32(seed, rng.STREAM_DRAWS, idx + 4) % np.uint32(33)).astype(np.int64)
    reqs = []
    for r in range(nreq):
        nr = int(n[r])
        if drafting[r]:
            comp = COMP_DROP if mode[r] == 0 else COMP_KIVI2
            reqs.append(Request(ctx_len=nr, x=int(step[r]) + 1, comp=comp,
                                recent=128 if comp == COMP_DROP else 0,
                                top=nr // 4 if comp == COMP_DROP else 0,
                                kind=KIND_DRAFT, step=int(step[r])))
        else:
            reqs.append(Request(ctx_len=nr, x=int(xv[r]), comp=COMP_DROP, recent=128,
                                top=nr // 4, kind=KIND_VERIFY))
    return Config("C5-ragged-mixed", cid, L=1, Hq=32, Hkv=8, d=128, reqs=reqs,
                  wu_width=4096, vocab=4096, mixed=True,
                  note="64 requests, lognormal n in [4K,128K], half draft (drop-4x or KIVI-2), "
                       "half verify x~U[8,40], one launch")


ALL = {
    "C1": c1_tiny,
    "C2": c2_llama8b_32k,
    "C3": c3_llama8b_100k_kivi2,
    "C4": c4_qwen32b_128k,
    "C5": c5_ragged,
}


def get(name: str) -> Config:
    return ALL[name]()


def scaled(cfg: Config, *, L: Optional[int] = None, B: Optional[int] = None,
           n: Optional[int] = None, x: Optional[int] = None, name_suffix: str = "-small") -> Config:
    """A smaller copy of a config (same head shape, compression kind and seed) for fast tests.

    Drop settings scale with n the way the full config defines them (R fixed, m = n // 4 for the
    4x drops; C1 keeps its fixed 64 + 192 unless n is smaller)."""
    reqs = []
    src = cfg.reqs if B is None else [cfg.reqs[i % len(cfg.reqs)] for i in range(B)]
    for r in src:
        nr = r.ctx_len if n is None else n
        xr = r.x if x is None else x
        rr = Request(ctx_len=nr, x=xr, comp=r.comp, recent=r.recent, top=r.top, kind=r.kind,
                     step=min(r.step, xr - 1))
        if n is not None and r.comp in (COMP_DROP, COMP_DROP_KIVI4):
            if cfg.cid == 1:
                rr.recent, rr.top = min(r.recent, nr), min(r.top, max(0, nr - r.recent))
            else:
                rr.recent, rr.top = min(r.recent, nr), nr // 4
        if r.kind == KIND_DRAFT:
            rr.x = rr.step + 1
        reqs.append(rr)
    return Config(cfg.name + name_suffix, cfg.cid, L=cfg.L if L is None else L, Hq=cfg.Hq,
                  Hkv=cfg.Hkv, d=cfg.d, reqs=reqs, wu_width=cfg.wu_width, vocab=cfg.vocab,
                  mixed=cfg.mixed, staged=cfg.staged, note=cfg.note + " (scaled)")


def page_permutation(seed: int, nblocks: int, salt: int) -> np.ndarray:
    """A seeded permutation of physical block ids [0, nblocks) (argsort of one u32 per block)."""
    keys = rng.u32(seed, rng.STREAM_PAGEPERM, np.arange(nblocks, dtype=np.int64) + (salt << 36))
    return np.argsort(keys, kind="stable").astype(np.int32)


def page_tables(seed: int, ntokens: List[int], salt: int, max_pages: Optional[int] = None):
    """Per-request page tables (int32 [B][max_pages], -1 = unused) over one shared block pool.

    Logical page p of request r gets physical block perm[offset_r + p]."""
    npages = [(t + BLOCK - 1) // BLOCK for t in ntokens]
    total = int(sum(npages))
    mp = max(npages) if max_pages is None else max_pages
    perm = page_permutation(seed, max(total, 1), salt)
    table = np.full((len(ntokens), max(mp, 1)), -1, dtype=np.int32)
    off = 0
    for r, p in enumerate(npages):
        table[r, :p] = perm[off:off + p]
        off += p
    return table, max(total, 1)
