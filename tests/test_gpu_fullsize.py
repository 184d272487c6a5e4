"""GPU path vs the fp64 oracle at the workloads' full sizes, in the launch configuration the
benchmark times (default split planning, x draft launches then one verify launch, logits and
accept), on sampled (request, layer, kv head) units the oracle computes one by one.

The sampled units' context rows are drawn by the seeded generator's GPU fill kernel (pinned
bit-exact against the CPU generator below); every expected value is the oracle's own float64
arithmetic.  Run on an MI355X: -m gpu.
"""
import gc

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, ctx_bits_gpu_generator, require_gpu, tight_tol, tokens_match
from oracle import accept as oacc
from oracle import attention as oatt
from oracle import workload as ow
from oracle.numerics import bf16_to_f64
from vcsynth import configs as C
from vcsynth import rng
from vcsynth import tensors as T

pytestmark = pytest.mark.gpu

# sampled (request, layer, kv head) units per workload
SAMPLES = {
    "C2": [(0, 0, 0), (3, 17, 5), (7, 31, 7)],
    "C3": [(0, 0, 0), (3, 31, 6)],
    "C4": [(0, 0, 0), (1, 63, 7)],
}
TOKEN_INSTANCE = {"C2": (7, 31)}  # (request, layer) whose logits, tokens and accept are checked


def _context(cfg, r, l, g):
    n = cfg.reqs[r].ctx_len
    return (bf16_to_f64(ctx_bits_gpu_generator(cfg, r, l, g, n, rng.STREAM_KCTX)),
            bf16_to_f64(ctx_bits_gpu_generator(cfg, r, l, g, n, rng.STREAM_VCTX)))


def _oracle_unit(cfg, r, l, g, x, q_all, steps=None, verify=True):
    """Verify rows [x][G][d] (None if not asked) and draft steps [len(steps)][G][d] (None if no
    steps) of one unit."""
    G = cfg.G
    kc, vc = _context(cfg, r, l, g)
    q = q_all[:, g * G:(g + 1) * G]
    kb, vb = ow.block(cfg, r, l, g, x)
    ver = oatt.verify_unit(q, kc, vc, kb, vb) if verify else None
    steps = list(range(x) if steps is None else steps)
    dr = None
    if steps:
        cm = ow.compressed(cfg, r, l, g, kc, vc)
        dr = np.stack([oatt.draft_unit(q[i], cm.k, cm.v, kb, vb, i) for i in steps])
    return ver, dr


def _run_full(name):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.get(name)
    print(f"building full-size {name}", flush=True)
    wl = Workload(cfg)
    wl.run_round()
    torch.cuda.synchronize()
    res = {"cfg": cfg, "units": {}, "inst": {}}
    for r, l, g in SAMPLES[name]:
        x = cfg.reqs[r].x
        sl = slice(g * cfg.G, (g + 1) * cfg.G)
        res["units"][(r, l, g)] = (wl.out_v[r, l, :x, sl].double().cpu().numpy(),
                                   wl.out_d[r, l, :x, sl].double().cpu().numpy())
    if name in TOKEN_INSTANCE:
        r, l = TOKEN_INSTANCE[name]
        inst = r * cfg.L + l
        x = cfg.reqs[r].x
        res["inst"] = {
            "tok_d": wl.tok_d[inst, :x].cpu().numpy(), "tok_v": wl.tok_v[inst, :x].cpu().numpy(),
            "acc": int(wl.acc_len[inst]), "next": int(wl.next_tok[inst]),
            "z_d": wl.z_d.view(cfg.B * cfg.L, wl.xmax, -1)[inst, :x].double().cpu().numpy(),
            "z_v": wl.z_v.view(cfg.B * cfg.L, wl.xmax, -1)[inst, :x].double().cpu().numpy()}
    del wl
    gc.collect()
    torch.cuda.empty_cache()
    return res


@pytest.fixture(scope="module", params=["C2", "C3", "C4"])
def full(request):
    return _run_full(request.param)


def test_gpu_generator_matches_cpu_at_full_strides():
    require_gpu()
    cfg = C.get("C4")
    n, p0 = 96, cfg.reqs[1].ctx_len - 96
    for stream, cpu in ((rng.STREAM_KCTX, T.kctx_bits), (rng.STREAM_VCTX, T.vctx_bits)):
        got = ctx_bits_gpu_generator(cfg, 1, 63, 7, n, stream, p0=p0)
        assert np.array_equal(got, cpu(cfg, 1, 63, 7, n, p0=p0))


def test_full_size_sampled_units(full):
    cfg = full["cfg"]
    for (r, l, g), (gv, gd) in full["units"].items():
        req = cfg.reqs[r]
        q_all = ow.queries(cfg, r, l, req.x)
        ver, dr = _oracle_unit(cfg, r, l, g, req.x, q_all)
        ev = assert_close(gv, ver, tight_tol(req.ctx_len), f"{cfg.name} verify r={r} l={l} g={g}")
        ed = assert_close(gd, dr, tight_tol(req.kept, kivi=req.bits != 16), f"{cfg.name} draft r={r} l={l} g={g}")
        print(f"{cfg.name} (r={r}, l={l}, g={g}): verify max-abs {ev:.2e}, draft max-abs {ed:.2e}")


def test_full_size_tokens_and_accept(full):
    cfg = full["cfg"]
    if cfg.name.split("-")[0] not in TOKEN_INSTANCE:
        pytest.skip("tokens are checked on one instance of the Llama-3.1-8B 32K workload")
    r, l = TOKEN_INSTANCE[cfg.name.split("-")[0]]
    x = cfg.reqs[r].x
    q_all = ow.queries(cfg, r, l, x)
    vo, do = [], []
    for g in range(cfg.Hkv):
        ver, dr = _oracle_unit(cfg, r, l, g, x, q_all)
        vo.append(ver)
        do.append(dr)
    vo, do = np.concatenate(vo, axis=1), np.concatenate(do, axis=1)   # [x][Hq][d]
    wu = bf16_to_f64(T.wu_bits(cfg))
    zv, zd = oacc.logits(vo.reshape(x, -1), wu), oacc.logits(do.reshape(x, -1), wu)
    tv, gv = oacc.argmax_gap(zv)
    td, gd = oacc.argmax_gap(zd)
    a, nxt = oacc.accept(td, tv)
    inst = full["inst"]
    assert not tokens_match(inst["tok_v"], tv, gv, zv)
    assert not tokens_match(inst["tok_d"], td, gd, zd)
    if not oacc.accept_flagged(a, x, gd, gv):
        assert (inst["acc"], inst["next"]) == (a, nxt)
    # the accept kernel on the GPU's own logits is exact
    td_g, _ = oacc.argmax_gap(inst["z_d"])
    tv_g, _ = oacc.argmax_gap(inst["z_v"])
    assert np.array_equal(inst["tok_d"], td_g) and np.array_equal(inst["tok_v"], tv_g)
    assert (inst["acc"], inst["next"]) == oacc.accept(td_g, tv_g)


def test_full_size_ragged_mixed_launch():
    """The 64-request ragged batch in one launch: sampled drafting (drop and KIVI-2) and
    verifying requests, two kv heads each."""
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.get("C5")
    wl = Workload(cfg)
    wl.run_mixed()
    torch.cuda.synchronize()
    ver = [r for r, q in enumerate(cfg.reqs) if q.kind == C.KIND_VERIFY]
    drop = [r for r, q in enumerate(cfg.reqs) if q.kind == C.KIND_DRAFT and q.comp == C.COMP_DROP]
    kivi = [r for r, q in enumerate(cfg.reqs) if q.kind == C.KIND_DRAFT and q.comp == C.COMP_KIVI2]
    by_len = lambda rs: [min(rs, key=lambda r: cfg.reqs[r].ctx_len), max(rs, key=lambda r: cfg.reqs[r].ctx_len)]
    picks = by_len(ver) + by_len(drop) + by_len(kivi)
    got = {r: wl.out_v[r, 0].double().cpu().numpy() for r in picks}
    del wl
    gc.collect()
    torch.cuda.empty_cache()
    G = cfg.G
    for r in picks:
        req = cfg.reqs[r]
        for g in (0, cfg.Hkv - 1):
            sl = slice(g * G, (g + 1) * G)
            if req.kind == C.KIND_VERIFY:
                ver_o, _ = _oracle_unit(cfg, r, 0, g, req.x, ow.queries(cfg, r, 0, req.x), steps=[])
                assert_close(got[r][:req.x, sl], ver_o, tight_tol(req.ctx_len), f"C5 verify r={r} g={g}")
            else:
                _, dr = _oracle_unit(cfg, r, 0, g, req.step + 1, ow.queries(cfg, r, 0, req.step + 1),
                                     steps=[req.step], verify=False)
                assert_close(got[r][req.step, sl], dr[0], tight_tol(req.kept, kivi=req.bits != 16),
                             f"C5 draft r={r} ({req.comp}, n={req.ctx_len}, step {req.step}) g={g}")


def test_staged_full_kv_verify_is_bit_identical():
    """The full KV of two layer slices of the Qwen-32B-like 128K workload is moved to pinned host
    memory, cleared on the device, and staged back with vc_stage_kv on a side stream while the
    draft steps run; the verify pass after the stream waits on the staging event must equal the
    verify over the resident cache bit for bit."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.get("C4")
    wl = Workload(cfg)
    wl.run_verify()
    torch.cuda.synchronize()
    layers = (0, cfg.L - 1)
    ref = {l: wl.out_v[:, l].clone() for l in layers}
    host = {}
    for l in layers:
        for name in ("k", "v"):
            dev = getattr(wl.full, name)[l]
            h = torch.empty(dev.shape, dtype=dev.dtype, pin_memory=True)
            h.copy_(dev)
            host[(l, name)] = h
            dev.zero_()
    wl.out_v.zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    staged = torch.cuda.Event(enable_timing=True)
    t0 = torch.cuda.Event(enable_timing=True)
    staged.record(side)   # creates the event; vc_stage_kv records it again after each copy
    t0.record(side)
    for (l, name), h in host.items():
        dev = getattr(wl.full, name)[l]
        vc.stage_kv(dev, h, dev.numel() * dev.element_size(), side, staged)
    for i in range(max(r.x for r in cfg.reqs)):   # drafts overlap the staging
        wl.run_draft(i)
    torch.cuda.current_stream().wait_event(staged)
    wl.run_verify()
    torch.cuda.synchronize()
    nbytes = sum(h.numel() * h.element_size() for h in host.values())
    print(f"staged {nbytes / 1e9:.2f} GB at {nbytes / t0.elapsed_time(staged) / 1e6:.1f} GB/s")
    for l in layers:
        assert torch.equal(wl.out_v[:, l], ref[l]), f"layer {l}"
    del wl, host
    gc.collect()
    torch.cuda.empty_cache()
