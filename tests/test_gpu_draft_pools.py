"""Mixed launches that hold only drafting requests, against the oracle (run on an MI355X: -m gpu).

vc_attn_mixed takes up to four pools and a pool index per request.  A launch without verifying
requests runs a draft kernel, which must be the one of its requests' pool kind whatever pool 0
is (here the bf16 full pool), and drafting requests over pools of two kinds (bf16 drop and
KIVI-2) must go to the kernel that picks the path per item.
"""
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def _cfg(kinds):
    D = C.KIND_DRAFT
    reqs = []
    for i, n in enumerate((700, 333, 1030, 481, 129, 900)):
        comp = kinds[i % len(kinds)]
        step = i % 5
        if comp == C.COMP_KIVI2:
            reqs.append(C.Request(ctx_len=n, x=step + 1, comp=comp, kind=D, step=step))
        else:
            reqs.append(C.Request(ctx_len=n, x=step + 1, comp=comp, recent=64, top=n // 4, kind=D, step=step))
    cid = {(C.COMP_DROP, C.COMP_KIVI2): 81, (C.COMP_KIVI2,): 82, (C.COMP_DROP,): 83}[tuple(kinds)]
    return C.Config(f"draft-only-{'-'.join(kinds)}", cid, L=1, Hq=16, Hkv=2, d=128, reqs=reqs, wu_width=2048,
                    vocab=1024, mixed=True)


@pytest.mark.parametrize("kinds", [(C.COMP_DROP, C.COMP_KIVI2), (C.COMP_KIVI2,), (C.COMP_DROP,)])
@pytest.mark.parametrize("split", [0, 4])
def test_draft_only_mixed_launch(kinds, split):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _cfg(list(kinds))
    print(f"draft-only mixed launch {kinds} split_pages={split}", flush=True)
    wl = Workload(cfg)
    reqs = wl.mixed_reqs()
    assert all(r.kind == vc.VC_DRAFT for r in reqs) and all(r.pool != 0 for r in reqs)
    wl.run_mixed(split)
    torch.cuda.synchronize()
    vc.check_device()
    for r, req in enumerate(cfg.reqs):
        want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
        got = wl.out_v[r, 0, req.step].double().cpu().numpy()
        assert_close(got, want[0], gate(spr[0], kivi=req.bits != 16),
                     f"draft-only r={r} ({req.comp}, step {req.step})")
