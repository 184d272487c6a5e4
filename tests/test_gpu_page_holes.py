"""Context pages whose page-table entry is -1, or names no block of the pool, contribute no keys:
every attention path against the oracle's attention over the remaining tokens (run on an
MI355X: -m gpu).  In a KIVI pool the key parameters of pages 2j and 2j+1 live in page 2j's
block, so a missing even page also removes its odd partner.  An entry past the pool is a corrupt
table, not a hole: the kernels also record it in the device error word, and vc_check_device()
reports it as VC_EDEVICE (once: the word is cleared by the read)."""
import re

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import attention as att
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def keep_mask(n: int, holes, kivi_pairs: bool = False) -> np.ndarray:
    """Tokens 0..n-1 that remain when the listed logical pages are missing."""
    keep = np.ones(n, dtype=bool)
    for p in holes:
        dropped = [p, p + 1] if (kivi_pairs and p % 2 == 0) else [p]
        for q in dropped:
            keep[16 * q:16 * (q + 1)] = False
    return keep


def punch(page_table: torch.Tensor, num_blocks: int, holes):
    """Mark pages missing: -1, except the last listed page of each row, which gets an id past the
    pool's blocks (also missing, and reported).  Returns the corrupt (row, page, id) entries."""
    bad = set()
    for r, pages in holes.items():
        for i, p in enumerate(pages):
            last = i == len(pages) - 1
            page_table[r, p] = num_blocks + 3 + r if last else -1
            if last:
                bad.add((r, p, num_blocks + 3 + r))
    return bad


def expect_reported(bad):
    """vc_check_device reports one of the corrupt entries, then nothing (the word is cleared)."""
    from lossless_kv_cache_vc_amd import vc
    with pytest.raises(vc.VCError) as e:
        vc.check_device()
    assert e.value.code == vc.VC_EDEVICE, str(e.value)
    m = re.search(r"row (\d+), logical page (\d+): block id (-?\d+)", str(e.value))
    assert m and tuple(int(v) for v in m.groups()) in bad, (str(e.value), bad)
    vc.check_device()


def test_holes_alone_report_nothing():
    """-1 entries are holes, not errors: a verify over a table with holes only leaves the error
    word clear."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get("C2"), L=1, B=2, n=500)
    wl = Workload(cfg, build_compressed=False)
    try:
        vc.check_device()   # whatever earlier work left
    except vc.VCError:
        pass
    wl.full.page_table[0, 3] = -1
    wl.full.page_table[1, 0] = -1
    wl.run_verify()
    vc.check_device()


@pytest.mark.parametrize("name,kw,split", [
    ("C2", dict(L=1, B=2, n=1000), 0),            # 128 rows: verify_kernel
    ("C2", dict(L=1, B=2, n=1000), 8),
    ("C4", dict(L=1, B=1, n=900, x=17), 0),       # 136 rows: verify_wide_kernel
    ("C4", dict(L=1, B=1, n=900, x=17), 8),
])
def test_verify_skips_missing_pages(name, kw, split):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get(name), **kw)
    print(f"verify holes {name} {kw} split={split}", flush=True)
    wl = Workload(cfg, build_compressed=False)
    holes = {0: [0, 3, 7, 8, 40], 1: [13, 60]} if cfg.B == 2 else {0: [1, 4, 5, 30, 56]}
    bad = punch(wl.full.page_table, wl.full.num_blocks, holes)
    wl.run_verify(split)
    torch.cuda.synchronize()
    expect_reported(bad)
    for r, req in enumerate(cfg.reqs):
        keep = keep_mask(req.ctx_len, holes.get(r, []))
        q = ow.queries(cfg, r, 0, req.x)
        for g in range(cfg.Hkv):
            kc, vc = ow.context(cfg, r, 0, g)
            kb, vb = ow.block(cfg, r, 0, g, req.x)
            want, spr = att.verify_unit(q[:, g * cfg.G:(g + 1) * cfg.G], kc[keep], vc[keep], kb, vb, spread=True)
            got = wl.out_v[r, 0, :req.x, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
            assert_close(got, want, gate(spr), f"verify holes r={r} g={g}")


@pytest.mark.parametrize("name,holes", [
    ("C2", {0: [2, 5, 23], 1: [0, 11]}),          # bf16 drop cache (kept tokens in pages)
    ("C3", {0: [5, 10, 62], 1: [0, 33]}),         # KIVI-2: odd page, even page (pair), the odd last page
    ("C4", {0: [3, 6, 23], 1: [0, 9]}),           # drop + KIVI-4 (4-bit ring, 24 kept pages)
])
def test_draft_skips_missing_pages(name, holes):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get(name), L=1, B=2, n=1000)
    print(f"draft holes {name}", flush=True)
    wl = Workload(cfg)
    pool = wl.drop_pool if wl.drop_pool is not None else wl.kivi_pool
    kivi = pool.bits != 16
    bad = punch(pool.page_table, pool.num_blocks, holes)
    steps = [0, 5]
    outs = {}
    for i in steps:
        wl.run_draft(i)
        torch.cuda.synchronize()
        outs[i] = wl.out_d.clone()
    expect_reported(bad)
    for r, req in enumerate(cfg.reqs):
        keep = keep_mask(wl.comp_len(r), holes.get(r, []), kivi_pairs=kivi)
        q = ow.queries(cfg, r, 0, max(steps) + 1)
        for g in range(cfg.Hkv):
            cm = ow.compressed(cfg, r, 0, g)
            kb, vb = ow.block(cfg, r, 0, g, max(steps) + 1)
            for i in steps:
                want, spr = att.draft_unit(q[i, g * cfg.G:(g + 1) * cfg.G], cm.k[keep], cm.v[keep], kb, vb, i,
                                           spread=True)
                got = outs[i][r, 0, i, g * cfg.G:(g + 1) * cfg.G].double().cpu().numpy()
                assert_close(got, want, gate(spr, kivi=kivi), f"draft holes r={r} g={g} i={i}")
