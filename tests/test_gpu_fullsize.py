"""GPU path vs the fp64 oracle at the workloads' full sizes, in the launch configuration the
benchmark times (default split planning, x draft launches then one verify launch, logits and
accept), on sampled (request, layer, kv head) units the oracle computes one by one.

The sampled units' context rows are drawn by the seeded generator's GPU fill kernel (pinned
bit-exact against the CPU generator below); every expected value is the oracle's own float64
arithmetic.  Run on an MI355X: -m gpu.
"""
import functools
import gc

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, ctx_bits_gpu_generator, gate, require_gpu, tokens_match
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
# (request, layer) whose logits, tokens and accept are checked against the oracle
TOKEN_INSTANCE = {"C2": (7, 31), "C3": (3, 31), "C4": (1, 63)}


def _context(cfg, r, l, g):
    n = cfg.reqs[r].ctx_len
    return (bf16_to_f64(ctx_bits_gpu_generator(cfg, r, l, g, n, rng.STREAM_KCTX)),
            bf16_to_f64(ctx_bits_gpu_generator(cfg, r, l, g, n, rng.STREAM_VCTX)))


def _oracle_unit(cfg, r, l, g, x, q_all, steps=None, verify=True):
    """(output, weight spread) of the verify rows [x][G][d] (None if not asked) and of the draft
    steps [len(steps)][G][d] (None if no steps) of one unit."""
    G = cfg.G
    kc, vc = _context(cfg, r, l, g)
    q = q_all[:, g * G:(g + 1) * G]
    kb, vb = ow.block(cfg, r, l, g, x)
    ver = oatt.verify_unit(q, kc, vc, kb, vb, spread=True) if verify else None
    steps = list(range(x) if steps is None else steps)
    dr = None
    if steps:
        cm = ow.compressed(cfg, r, l, g, kc, vc)
        res = [oatt.draft_unit(q[i], cm.k, cm.v, kb, vb, i, spread=True) for i in steps]
        dr = (np.stack([a for a, _ in res]), np.stack([b for _, b in res]))
    return ver, dr


def _units(wl, cfg, name, out):
    got = {}
    for r, l, g in SAMPLES[name]:
        x = cfg.reqs[r].x
        sl = slice(g * cfg.G, (g + 1) * cfg.G)
        got[(r, l, g)] = out[r, l, :x, sl].double().cpu().numpy()
    return got


def _stage_and_verify(wl, cfg):
    """The full cache's row of the workload (it lives in pinned host memory and is reloaded into
    HBM on a side stream while the drafter runs): copy the whole full pool to exact-size pinned
    host buffers, clear it on the device, reload every layer slice with vc_stage_kv on a side
    stream while the x draft launches run on the compute stream, make the compute stream wait on
    the staging event, and run the verify over the reloaded pool."""
    bufs = wl.full_to_host()
    wl.full.k.zero_()
    wl.full.v.zero_()
    out = torch.full_like(wl.out_v, float("nan"))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    t0 = torch.cuda.Event(enable_timing=True)
    staged = torch.cuda.Event(enable_timing=True)
    t0.record(side)
    nbytes = wl.stage_full(bufs, side, staged)
    for i in range(max(r.x for r in cfg.reqs)):   # the draft steps overlap the reload
        wl.run_draft(i)
    torch.cuda.current_stream().wait_event(staged)
    wl.run_verify(out=out)
    torch.cuda.synchronize()
    gbps = nbytes / (t0.elapsed_time(staged) * 1e-3) / 1e9
    print(f"staged {nbytes / 1e9:.1f} GB at {gbps:.1f} GB/s", flush=True)
    del bufs
    return out, nbytes, gbps


@functools.lru_cache(maxsize=3)
def _run_full(name):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.get(name)
    print(f"building full-size {name}", flush=True)
    wl = Workload(cfg)
    wl.run_round()
    torch.cuda.synchronize()
    res = {"cfg": cfg, "inst": {}}
    ver, dr = _units(wl, cfg, name, wl.out_v), _units(wl, cfg, name, wl.out_d)
    res["units"] = {u: (ver[u], dr[u]) for u in ver}
    r, l = TOKEN_INSTANCE[name]
    inst = r * cfg.L + l
    x = cfg.reqs[r].x
    res["inst"] = {
        "tok_d": wl.tok_d[inst, :x].cpu().numpy(), "tok_v": wl.tok_v[inst, :x].cpu().numpy(),
        "acc": int(wl.acc_len[inst]), "next": int(wl.next_tok[inst]),
        "z_d": wl.z_d.view(cfg.B * cfg.L, wl.xmax, -1)[inst, :x].double().cpu().numpy(),
        "z_v": wl.z_v.view(cfg.B * cfg.L, wl.xmax, -1)[inst, :x].double().cpu().numpy()}
    if cfg.staged:
        resident = wl.out_v.clone()
        out, nbytes, gbps = _stage_and_verify(wl, cfg)
        x = cfg.reqs[0].x   # every request verifies x rows; rows past x are not written
        same = torch.equal(out[:, :, :x].view(torch.int32), resident[:, :, :x].view(torch.int32))
        res["staged"] = {"units": _units(wl, cfg, name, out), "bytes": nbytes, "gbps": gbps,
                         "identical": bool(same)}
        del out, resident
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
        (ver, vspr), (dr, dspr) = _oracle_unit(cfg, r, l, g, req.x, q_all)
        ev = assert_close(gv, ver, gate(vspr), f"{cfg.name} verify r={r} l={l} g={g}")
        ed = assert_close(gd, dr, gate(dspr, kivi=req.bits != 16), f"{cfg.name} draft r={r} l={l} g={g}")
        print(f"{cfg.name} (r={r}, l={l}, g={g}): verify max-abs {ev:.2e}, draft max-abs {ed:.2e}")


def test_full_size_tokens_and_accept(full):
    cfg = full["cfg"]
    r, l = TOKEN_INSTANCE[cfg.name.split("-")[0]]
    x = cfg.reqs[r].x
    q_all = ow.queries(cfg, r, l, x)
    vo, do = [], []
    for g in range(cfg.Hkv):
        (ver, _), (dr, _) = _oracle_unit(cfg, r, l, g, x, q_all)
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
                (ver_o, vspr), _ = _oracle_unit(cfg, r, 0, g, req.x, ow.queries(cfg, r, 0, req.x), steps=[])
                assert_close(got[r][:req.x, sl], ver_o, gate(vspr), f"C5 verify r={r} g={g}")
            else:
                _, (dr, dspr) = _oracle_unit(cfg, r, 0, g, req.step + 1, ow.queries(cfg, r, 0, req.step + 1),
                                             steps=[req.step], verify=False)
                assert_close(got[r][req.step, sl], dr[0], gate(dspr[0], kivi=req.bits != 16),
                             f"C5 draft r={r} ({req.comp}, n={req.ctx_len}, step {req.step}) g={g}")


def test_staged_full_kv_verify_matches_the_oracle():
    """The Qwen-32B-like 128K workload with its full KV (68.7 GB, every layer slice) reloaded from
    pinned host memory on a side stream while the 40 draft launches run: the verify over the
    reloaded pool equals the resident verify bit for bit, and its sampled units match the oracle."""
    res = _run_full("C4")
    cfg = res["cfg"]
    st = res["staged"]
    assert st["bytes"] >= cfg.full_kv_bytes()
    assert st["identical"], "verify after the reload differs from the resident verify"
    for (r, l, g), got in st["units"].items():
        req = cfg.reqs[r]
        (ver, vspr), _ = _oracle_unit(cfg, r, l, g, req.x, ow.queries(cfg, r, l, req.x), steps=[])
        e = assert_close(got, ver, gate(vspr), f"staged verify r={r} l={l} g={g}")
        print(f"staged (r={r}, l={l}, g={g}): verify max-abs {e:.2e}; reload {st['gbps']:.1f} GB/s")
