"""Head dim 64 on the KIVI draft paths and in a mixed launch, against the oracle.

The five workloads use d = 128 for every KIVI cache (C1, the only d = 64 one, is bf16), but the
library takes d = 64 on every path.  Its KIVI ring slots have their own shapes (16- or 32-byte
key rows, interleaved with the other page in 128-byte blocks), so they are checked here: every
draft step of 2-bit and drop + 4-bit launches, and mixed launches that hold bf16 and KIVI
drafting requests beside verifying requests, one of them with two row groups.
"""
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def _kivi_cfg(comp):
    # contexts with a ragged last key group, an odd last page (outside the ring) and an exact
    # multiple of the 32-token group; G = 4, two layer slices
    def req(n):
        if comp == C.COMP_KIVI2:
            return C.Request(ctx_len=n, x=6, comp=comp)
        return C.Request(ctx_len=n, x=6, comp=comp, recent=64, top=n // 4)
    cid = 61 if comp == C.COMP_KIVI2 else 62
    return C.Config(f"d64-{comp}", cid, L=2, Hq=8, Hkv=2, d=64, reqs=[req(777), req(333), req(1024)],
                    wu_width=512, vocab=1024)


@pytest.mark.parametrize("comp", [C.COMP_KIVI2, C.COMP_DROP_KIVI4])
def test_kivi_draft_parity_head_dim_64(comp):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _kivi_cfg(comp)
    print(f"d=64 draft {comp}", flush=True)
    wl = Workload(cfg)
    for i in range(max(r.x for r in cfg.reqs)):
        wl.run_draft(i)
    torch.cuda.synchronize()
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            cc = [ow.compressed(cfg, r, l, g) for g in range(cfg.Hkv)]
            want, spr = ow.draft_out(cfg, r, l, range(req.x), comp_cache=cc, spread=True)
            got = wl.out_d[r, l, :req.x].double().cpu().numpy()
            worst = max(worst, assert_close(got, want, gate(spr, kivi=True),
                                            f"d64 {comp} draft r={r} l={l}"))
    print(f"d=64 {comp} draft max-abs error {worst:.3e}")


def _mixed_cfg(kivi):
    """A ragged launch at d = 64: bf16 and KIVI drafting requests (the harness builds one KIVI
    bit width per workload) beside verifying ones, one of which has 160 rows (two row groups
    that share its K/V)."""
    D, V = C.KIND_DRAFT, C.KIND_VERIFY

    def kreq(n, step):
        if kivi == C.COMP_KIVI2:
            return C.Request(ctx_len=n, x=step + 1, comp=kivi, kind=D, step=step)
        return C.Request(ctx_len=n, x=step + 1, comp=kivi, recent=64, top=n // 4, kind=D, step=step)
    reqs = [
        C.Request(ctx_len=900, x=40, comp=C.COMP_DROP, recent=64, top=900 // 4, kind=V),  # 160 rows
        C.Request(ctx_len=613, x=8, comp=C.COMP_DROP, recent=64, top=613 // 4, kind=V),
        kreq(700, 3),
        C.Request(ctx_len=555, x=2, comp=C.COMP_DROP, recent=64, top=555 // 4, kind=D, step=1),
        kreq(481, 0),
        kreq(1030, 4),
    ]
    cid = 63 if kivi == C.COMP_KIVI2 else 64
    return C.Config(f"d64-mixed-{kivi}", cid, L=1, Hq=8, Hkv=2, d=64, reqs=reqs, wu_width=512,
                    vocab=1024, mixed=True)


@pytest.mark.parametrize("kivi", [C.COMP_KIVI2, C.COMP_DROP_KIVI4])
def test_mixed_parity_head_dim_64(kivi):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _mixed_cfg(kivi)
    print(f"d=64 mixed launch ({kivi} drafts)", flush=True)
    wl = Workload(cfg)
    wl.run_mixed()
    torch.cuda.synchronize()
    for r, req in enumerate(cfg.reqs):
        if req.kind == C.KIND_VERIFY:
            want, spr = ow.verify_out(cfg, r, 0, spread=True)
            got = wl.out_v[r, 0, :req.x].double().cpu().numpy()
            assert_close(got, want, gate(spr), f"d64 mixed verify r={r}")
        else:
            want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
            want, spr = want[0], spr[0]
            got = wl.out_v[r, 0, req.step].double().cpu().numpy()
            assert_close(got, want, gate(spr, kivi=req.bits != 16),
                         f"d64 mixed draft r={r} ({req.comp}, step {req.step})")
