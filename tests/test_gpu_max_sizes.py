"""Launches at the boundary's limits, against the oracle (run on an MI355X: -m gpu).

* VC_MAX_REQS = 1024 requests in one mixed launch (the request table in the workspace, the
  ballot search over all of it), unsplit and with context splits merged from the same table;
* VC_MAX_ROWS = 64 drafted rows with G = 16 query heads per kv head: 1024 query rows per
  (layer, kv head) in one verify launch (four 256-row groups sharing their K/V), unsplit and split.
"""
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def ragged(nreq: int, cut: int) -> C.Config:
    cfg = C.c5_ragged(nreq)
    for r in cfg.reqs:
        r.ctx_len = max(40, r.ctx_len // cut)
        if r.comp == C.COMP_DROP:
            r.top = r.ctx_len // 4
    return cfg


@pytest.mark.parametrize("split", [0, 4])
def test_mixed_launch_of_the_maximum_request_count(split):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = ragged(vc.MAX_REQS, 400)
    print(f"mixed launch of {len(cfg.reqs)} requests, split_pages={split}", flush=True)
    wl = Workload(cfg)
    wl.run_mixed(split)
    torch.cuda.synchronize()
    vc.check_device()
    for r, req in enumerate(cfg.reqs):
        if req.kind == C.KIND_VERIFY:
            want, spr = ow.verify_out(cfg, r, 0, spread=True)
            got = wl.out_v[r, 0, :req.x].double().cpu().numpy()
            assert_close(got, want, gate(spr), f"mixed1024 verify r={r}")
        else:
            want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
            want, spr = want[0], spr[0]
            got = wl.out_v[r, 0, req.step].double().cpu().numpy()
            assert_close(got, want, gate(spr, kivi=req.bits != 16), f"mixed1024 draft r={r}")


@pytest.mark.parametrize("split", [0, 8])
def test_verify_of_the_maximum_row_count(split):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    x = vc.MAX_ROWS
    reqs = [C.Request(ctx_len=613, x=x, comp=C.COMP_DROP, recent=64, top=613 // 4),
            C.Request(ctx_len=190, x=x, comp=C.COMP_DROP, recent=64, top=190 // 4)]
    cfg = C.Config("max-rows-g16", 45, L=1, Hq=32, Hkv=2, d=128, reqs=reqs, wu_width=4096, vocab=1024)
    assert cfg.G * x == 1024
    print(f"verify of {cfg.G * x} rows per kv head, split_pages={split}", flush=True)
    wl = Workload(cfg)
    wl.run_verify(split)
    wl.run_draft(x - 1, split)
    torch.cuda.synchronize()
    vc.check_device()
    for r, req in enumerate(cfg.reqs):
        want, spr = ow.verify_out(cfg, r, 0, spread=True)
        got = wl.out_v[r, 0, :x].double().cpu().numpy()
        assert_close(got, want, gate(spr), f"max-rows verify r={r}")
        cc = [ow.compressed(cfg, r, 0, g) for g in range(cfg.Hkv)]
        want, spr = ow.draft_out(cfg, r, 0, [x - 1], comp_cache=cc, spread=True)
        want, spr = want[0], spr[0]
        got = wl.out_d[r, 0, x - 1].double().cpu().numpy()
        assert_close(got, want, gate(spr), f"max-rows draft r={r} (step {x - 1})")
