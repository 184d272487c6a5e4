"""The C ABI's boundary behaviour on the GPU (run on an MI355X: -m gpu):

* launches of more than 64 requests, whose request table lives in the workspace, against the
  oracle: a ragged batch of drafting and verifying requests in one mixed launch, and verify and
  draft launches with context splits (the merge kernel finds its requests in the same table);
* vc_stage_kv refuses a pageable source or a host destination, and records its event even when
  there is nothing to copy;
* the cache builder never writes through a corrupt page-table entry, and reports it.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def ragged(nreq: int) -> C.Config:
    """The ragged mixed batch with nreq requests, context lengths cut 40-fold (at least 90) so the
    oracle checks every output."""
    cfg = C.c5_ragged(nreq)
    for r in cfg.reqs:
        r.ctx_len = max(90, r.ctx_len // 40)
        if r.comp == C.COMP_DROP:
            r.top = r.ctx_len // 4
    return cfg


@pytest.mark.parametrize("nreq,split", [(96, 0), (96, 8), (160, 0)])
def test_mixed_launch_of_more_than_64_requests(nreq, split):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = ragged(nreq)
    print(f"mixed launch of {nreq} requests, split_pages={split}", flush=True)
    wl = Workload(cfg)
    assert vc.attn_workspace_size(wl.shape, wl.mixed_reqs(), split) >= nreq * 56
    wl.run_mixed(split)
    torch.cuda.synchronize()
    vc.check_device()
    for r, req in enumerate(cfg.reqs):
        if req.kind == C.KIND_VERIFY:
            want, spr = ow.verify_out(cfg, r, 0, spread=True)
            got = wl.out_v[r, 0, :req.x].double().cpu().numpy()
            assert_close(got, want, gate(spr), f"mixed{nreq} verify r={r}")
        else:
            want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
            want, spr = want[0], spr[0]
            got = wl.out_v[r, 0, req.step].double().cpu().numpy()
            assert_close(got, want, gate(spr, kivi=req.bits != 16), f"mixed{nreq} draft r={r}")


@pytest.mark.parametrize("split", [0, 4])
def test_verify_and_draft_launches_of_more_than_64_requests(split):
    """80 requests of the 8B shape (one layer, 300 tokens): the verify and a draft step, unsplit
    and with splits of 4 pages (5 splits per request, merged)."""
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get("C2"), L=1, B=80, n=300, x=8)
    print(f"80-request verify and draft, split_pages={split}", flush=True)
    wl = Workload(cfg)
    wl.run_verify(split)
    wl.run_draft(3, split)
    torch.cuda.synchronize()
    for r, req in enumerate(cfg.reqs):
        want, spr = ow.verify_out(cfg, r, 0, spread=True)
        assert_close(wl.out_v[r, 0, :req.x].double().cpu().numpy(), want, gate(spr),
                     f"verify80 r={r}")
        want, spr = ow.draft_out(cfg, r, 0, [3], spread=True)
        want, spr = want[0], spr[0]
        assert_close(wl.out_d[r, 0, 3].double().cpu().numpy(), want, gate(spr), f"draft80 r={r}")


def test_stage_kv_rejects_pageable_memory_and_records_its_event():
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    n = 1 << 20
    dev = torch.zeros(n, dtype=torch.uint8, device="cuda")
    pageable = np.arange(n, dtype=np.uint64).astype(np.uint8)
    lib = vc.lib()
    side = torch.cuda.Stream()
    rc = lib.vc_stage_kv(dev.data_ptr(), pageable.ctypes.data, n, side.cuda_stream, None)
    assert rc == vc.VC_EINVAL and "pinned" in vc.lib().vc_last_error().decode()
    pinned = torch.from_numpy(pageable).pin_memory()
    host_dst = torch.empty(n, dtype=torch.uint8).pin_memory()
    rc = lib.vc_stage_kv(host_dst.data_ptr(), pinned.data_ptr(), n, side.cuda_stream, None)
    assert rc == vc.VC_EINVAL and "device memory" in vc.lib().vc_last_error().decode()
    ev = torch.cuda.Event()
    ev.record(side)   # torch creates the HIP event on its first record
    vc.stage_kv(dev, pinned, n, side, ev)
    torch.cuda.current_stream().wait_event(ev)
    torch.cuda.synchronize()
    assert torch.equal(dev.cpu(), pinned)
    # nothing to copy: the event is still recorded (after the work already on the side stream)
    ev2 = torch.cuda.Event()
    ev2.record(torch.cuda.current_stream())
    vc.stage_kv(dev, pinned, 0, side, ev2)
    ev2.synchronize()
    assert ev2.query()


def test_pack_never_writes_through_a_corrupt_entry():
    """Page-table rows with a hole (-1) and an id past the pool: those pages are not written
    (the pool keeps its sentinel), every other page is, and the corrupt entry is reported."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    L, Hkv, d, n = 1, 2, 64, 80       # 5 pages
    nblk = 8
    shp = vc.shape(L, 8, Hkv, d, 16)
    pt = torch.tensor([[3, -1, 0, nblk + 5, 6]], dtype=torch.int32, device="cuda")
    k = torch.full((L, nblk, Hkv, 16, d), 7.0, dtype=torch.bfloat16, device="cuda")
    v = torch.full((L, nblk, Hkv, 16, d), 7.0, dtype=torch.bfloat16, device="cuda")
    pool = vc.PagedPool(16, pt, k, v, nblk)
    src = torch.randn((1, Hkv, n, d), dtype=torch.float32, device="cuda").to(torch.bfloat16)
    try:
        vc.check_device()
    except vc.VCError:
        pass
    vc.pack_bf16(shp, [n], 0, src, n, pool, 0)
    with pytest.raises(vc.VCError) as e:
        vc.check_device()
    assert e.value.code == vc.VC_EDEVICE and f"logical page 3: block id {nblk + 5}" in str(e.value)
    kk = k.float().cpu()
    ss = src.float().cpu()
    for p, b in enumerate([3, -1, 0, nblk + 5, 6]):
        if 0 <= b < nblk:
            assert torch.equal(kk[0, b], ss[0, :, 16 * p:16 * p + 16]), p
    for b in (1, 2, 4, 5, 7):   # never named by a valid entry
        assert torch.all(kk[0, b] == 7.0), b


def test_guard_regions_catch_a_write_past_a_tensor():
    """The guard regions the harness puts around every written tensor (VC_CANARY=1 in the tests)
    report a changed byte: one guard byte is overwritten from the host (a torch write into the
    guard, no kernel involved), the check must fail, and pass again once it is restored."""
    require_gpu()
    from lossless_kv_cache_vc_amd import harness
    from lossless_kv_cache_vc_amd.harness import Workload
    assert harness._canary_on(), "the tests run with guard regions"
    cfg = C.scaled(C.get("C2"), L=1, B=1, n=200, x=8)
    wl = Workload(cfg, build_compressed=False)
    wl.run_verify()
    wl.check_canaries()
    buf, n = wl._guards[-1]
    buf[harness.CANARY_BYTES + n + 7] = 0          # just past the end of that tensor
    with pytest.raises(AssertionError, match="1 after it"):
        wl.check_canaries()
    buf[harness.CANARY_BYTES + n + 7] = harness.CANARY_BYTE
    wl.check_canaries()
