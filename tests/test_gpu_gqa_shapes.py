"""Query-head grouping beyond the workloads' G = 4 and 8, against the oracle.

G = 1 (one query head per kv head: a draft row fills one of the 16 MFMA columns), G = 2 and G = 16
(a draft step fills all 16 columns; a verify position is 16 rows), each with bf16-drop, 2-bit KIVI
and drop + 4-bit KIVI drafting caches, at d = 64 and d = 128.  Every draft step and every verify
row is compared with the oracle.
"""
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu

CASES = [(1, 128, C.COMP_DROP), (1, 64, C.COMP_KIVI2), (2, 128, C.COMP_DROP_KIVI4),
         (2, 64, C.COMP_DROP), (16, 128, C.COMP_KIVI2), (16, 64, C.COMP_DROP_KIVI4),
         (16, 128, C.COMP_DROP)]


def _cfg(G, d, comp):
    Hkv = 2
    def req(n, x):
        if comp == C.COMP_KIVI2:
            return C.Request(ctx_len=n, x=x, comp=comp)
        return C.Request(ctx_len=n, x=x, comp=comp, recent=64, top=n // 4)
    cid = 70 + CASES.index((G, d, comp))
    # x * G stays at most 128 rows for G = 16 (8 positions); ragged context tails
    x = 8 if G == 16 else 12
    return C.Config(f"gqa{G}-d{d}-{comp}", cid, L=2, Hq=G * Hkv, Hkv=Hkv, d=d,
                    reqs=[req(611, x), req(290, x)], wu_width=G * Hkv * d, vocab=1024)


@pytest.mark.parametrize("G,d,comp", CASES)
def test_draft_and_verify_parity_gqa(G, d, comp):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _cfg(G, d, comp)
    print(f"G={G} d={d} {comp}", flush=True)
    wl = Workload(cfg)
    for i in range(max(r.x for r in cfg.reqs)):
        wl.run_draft(i)
    wl.run_verify()
    torch.cuda.synchronize()
    worst_d = worst_v = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            cc = [ow.compressed(cfg, r, l, g) for g in range(cfg.Hkv)]
            want, spr = ow.draft_out(cfg, r, l, range(req.x), comp_cache=cc, spread=True)
            got = wl.out_d[r, l, :req.x].double().cpu().numpy()
            worst_d = max(worst_d, assert_close(got, want, gate(spr, kivi=req.bits != 16),
                                                f"G={G} d={d} {comp} draft r={r} l={l}"))
            want, spr = ow.verify_out(cfg, r, l, spread=True)
            got = wl.out_v[r, l, :req.x].double().cpu().numpy()
            worst_v = max(worst_v, assert_close(got, want, gate(spr),
                                                f"G={G} d={d} {comp} verify r={r} l={l}"))
    print(f"G={G} d={d} {comp}: draft max-abs {worst_d:.3e}, verify {worst_v:.3e}")
