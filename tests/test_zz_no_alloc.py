"""vc_attn_mixed_noalloc, the attention launch whose workspace is the library's own device array,
against vc_attn_mixed with a caller workspace (run on an MI355X: -m gpu).

Two calls in a row through the C ABI, the second with a smaller input, each checked bit for bit
against vc_attn_mixed on the same arguments (the same kernels and plan) and on sampled requests
against the oracle: the array keeps the first call's request table and split partials, and the
second call must not read any of them.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def ragged(nreq: int) -> C.Config:
    """The ragged mixed batch with nreq requests, context lengths cut 40-fold (at least 90)."""
    cfg = C.c5_ragged(nreq)
    for r in cfg.reqs:
        r.ctx_len = max(90, r.ctx_len // 40)
        if r.comp == C.COMP_DROP:
            r.top = r.ctx_len // 4
    return cfg


def _check(cfg, wl, split):
    from lossless_kv_cache_vc_amd import vc
    reqs, pools = wl.mixed_reqs(), wl.mixed_pools()
    need = vc.attn_workspace_size(wl.shape, reqs, split)
    assert 0 < need <= vc.SCRATCH_BYTES
    ws = torch.empty(need // 4 + 1, dtype=torch.float32, device="cuda")
    ref = torch.full_like(wl.out_v, float("nan"))
    got = torch.full_like(wl.out_v, float("nan"))
    vc.attn_mixed(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pools, ref, ws, split)
    vc.attn_mixed_noalloc(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pools, got, split)
    torch.cuda.synchronize()
    vc.check_device()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), "outputs differ from vc_attn_mixed"
    picks = [0, 1, len(cfg.reqs) // 2, len(cfg.reqs) - 1]
    for r in picks:
        req = cfg.reqs[r]
        if req.kind == C.KIND_VERIFY:
            want, spr = ow.verify_out(cfg, r, 0, spread=True)
            assert_close(got[r, 0, :req.x].double().cpu().numpy(), want, gate(spr),
                         f"noalloc verify r={r}")
        else:
            want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
            want, spr = want[0], spr[0]
            assert_close(got[r, 0, req.step].double().cpu().numpy(), want,
                         gate(spr, kivi=req.bits != 16), f"noalloc draft r={r}")


def test_noalloc_matches_the_workspace_launch_twice():
    """First a 96-request launch split 16 pages at a time (request table and split partials:
    61.7 MiB of the 64 MiB array), then a 24-request one split 4 pages at a time (partials only,
    35.8 MiB, laid out differently)."""
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    for nreq, split in ((96, 16), (24, 4)):
        print(f"noalloc mixed launch of {nreq} requests, split_pages={split}", flush=True)
        cfg = ragged(nreq)
        wl = Workload(cfg)
        _check(cfg, wl, split)
        del wl
        torch.cuda.empty_cache()


def test_noalloc_refuses_launches_beyond_its_array():
    """A launch whose workspace would exceed the array is refused before anything is enqueued:
    the output keeps its contents."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get("C2"), L=1, B=2, n=2000, x=8)
    wl = Workload(cfg, build_compressed=False)
    reqs = [vc.Req(r, 0, cfg.reqs[r].ctx_len, r, 0, cfg.reqs[r].x, vc.VC_VERIFY) for r in range(cfg.B)]
    # splits of 4 pages: 32 splits x 8 kv heads x 32 rows x 132 floats = 4.3 MB of partials per
    # request, so 1024 requests (the launch limit) need about 4.4 GB
    many = reqs * 512
    need = vc.attn_workspace_size(wl.shape, many, 4)
    assert need > vc.SCRATCH_BYTES
    sentinel = torch.full_like(wl.out_v, 3.0)
    with pytest.raises(vc.VCError) as e:
        vc.attn_mixed_noalloc(wl.shape, many, wl.q, wl.blk_k, wl.blk_v, [wl.full], sentinel, 4)
    assert e.value.code == vc.VC_ENOSPACE
    torch.cuda.synchronize()
    assert torch.all(sentinel == 3.0)
