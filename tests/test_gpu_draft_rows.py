"""Draft launches whose requests carry several query rows, against the oracle (run on an MI355X: -m gpu).

A drafting request covers block positions q0 .. q0 + rows - 1 (rows * G <= 16 query rows per kv
head); position j sees the compressed context and drafted rows 0 .. j, as the j-th draft step does
on its own.  The cases put 3 or 4 rows (G = 1, 2 and 3: the layout that repeats the rows over four
column slots), 6, 8 and 16 rows per kv head in one step, over each drafting cache kind, and
compare every row with the oracle's single steps.
"""
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu

# (G, rows per request, head dim, drafting cache)
CASES = [(1, 4, 128, C.COMP_KIVI2), (2, 2, 128, C.COMP_DROP_KIVI4), (2, 2, 64, C.COMP_KIVI2),
         (1, 3, 128, C.COMP_DROP), (2, 3, 128, C.COMP_KIVI2), (4, 2, 128, C.COMP_DROP_KIVI4),
         (4, 4, 128, C.COMP_DROP), (4, 4, 64, C.COMP_KIVI2),
         # 3 rows per kv head: one column of each 4-column slot holds no row
         (1, 3, 128, C.COMP_KIVI2), (3, 1, 128, C.COMP_DROP_KIVI4)]


def _cfg(G, d, comp, case):
    Hkv = 2

    def req(n):
        if comp == C.COMP_KIVI2:
            return C.Request(ctx_len=n, x=8, comp=comp)
        return C.Request(ctx_len=n, x=8, comp=comp, recent=64, top=n // 4)
    return C.Config(f"draft-rows-g{G}-d{d}-{comp}", 100 + case, L=2, Hq=G * Hkv, Hkv=Hkv, d=d,
                    reqs=[req(611), req(290)], wu_width=G * Hkv * d, vocab=1024)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_multi_row_draft_parity(case):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    G, rows, d, comp = CASES[case]
    cfg = _cfg(G, d, comp, case)
    print(f"multi-row draft: G={G} rows={rows} d={d} {comp}", flush=True)
    wl = Workload(cfg)
    pool = wl.drop_pool if wl.drop_pool is not None else wl.kivi_pool
    # two launches: positions 0 .. rows - 1, then a later window ending at the last drafted row
    windows = [0, cfg.reqs[0].x - rows]
    for q0 in windows:
        reqs = [vc.Req(r, 0, wl.comp_len(r), r, q0, rows, vc.VC_DRAFT) for r in range(cfg.B)]
        need = vc.attn_workspace_size(wl.shape, reqs)
        ws = torch.empty(need // 4 + 1, dtype=torch.float32, device=wl.out_d.device) if need else None
        vc.draft_attn(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pool, wl.out_d, ws, 0)
    torch.cuda.synchronize()
    vc.check_device()
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            cc = [ow.compressed(cfg, r, l, g) for g in range(cfg.Hkv)]
            for q0 in windows:
                want, spr = ow.draft_out(cfg, r, l, range(q0, q0 + rows), comp_cache=cc, spread=True)
                got = wl.out_d[r, l, q0:q0 + rows].double().cpu().numpy()
                worst = max(worst, assert_close(got, want, gate(spr, kivi=req.bits != 16),
                                                f"G={G} rows={rows} d={d} {comp} r={r} l={l} q0={q0}"))
    print(f"G={G} rows={rows} d={d} {comp}: max-abs {worst:.3e}")
