"""Attention launches recorded in a HIP graph and replayed (run on an MI355X: -m gpu).

Callers under graph capture cannot allocate; vc_attn_mixed_noalloc takes its workspace from the
library's own device array, and vc_attn_mixed takes one the caller allocated before capture.
A ragged mixed batch of 80 requests (so the request table is written into the workspace by upload
kernels, which the graph records too) split 16 pages at a time (split partials and the merge) is
captured once through each entry point and replayed three times, with eager work on the outputs
and synchronisations between the replays; every replay must equal the eager launch bit for bit.
The library makes no allocating, copying or synchronising runtime call on these paths (the
device array's address is looked up by the first call, made eagerly here).
"""
import pytest
import torch

from gpu_helpers import require_gpu
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def _ragged(nreq):
    cfg = C.c5_ragged(nreq)
    for r in cfg.reqs:
        r.ctx_len = max(90, r.ctx_len // 40)
        if r.comp == C.COMP_DROP:
            r.top = r.ctx_len // 4
    return cfg


def test_mixed_launches_replay_from_a_graph():
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _ragged(80)
    wl = Workload(cfg)
    reqs, pools = wl.mixed_reqs(), wl.mixed_pools()
    split = 16
    need = vc.attn_workspace_size(wl.shape, reqs, split)
    assert 0 < need <= vc.SCRATCH_BYTES
    ws = torch.empty(need // 4 + 1, dtype=torch.float32, device="cuda")
    ref = torch.full_like(wl.out_v, float("nan"))
    vc.attn_mixed_noalloc(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pools, ref, split)
    torch.cuda.synchronize()
    vc.check_device()

    out_n = torch.full_like(wl.out_v, float("nan"))
    out_w = torch.full_like(wl.out_v, float("nan"))
    side = torch.cuda.Stream()
    g_n, g_w = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_n, stream=side):
        vc.attn_mixed_noalloc(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pools, out_n, split, stream=side)
    with torch.cuda.graph(g_w, stream=side):
        vc.attn_mixed(wl.shape, reqs, wl.q, wl.blk_k, wl.blk_v, pools, out_w, ws, split, stream=side)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: refill the outputs as the reference was initialised (the
        # launches write only their requests' rows)
        out_n.fill_(float("nan"))
        out_w.fill_(float("nan"))
        torch.cuda.synchronize()
        g_n.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_n.view(torch.int32), ref.view(torch.int32)), f"no-alloc replay {rep}"
        g_w.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_w.view(torch.int32), ref.view(torch.int32)), f"workspace replay {rep}"
    vc.check_device()
