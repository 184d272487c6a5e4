"""GPU path vs the fp64 oracle on identical seeded inputs (run on an MI355X: -m gpu).

Scaled configs keep each workload's head shape, compression kind and seed but use fewer layers,
requests and tokens, so the oracle checks every output element; sizes still span several
64-key tiles and end on a ragged page.  Full-size configs are checked on sampled (request,
layer, kv head) units in the launch configuration the benchmark times.
"""
import functools

import numpy as np
import pytest
import torch

from gpu_helpers import (assert_close, pool_kivi, pool_tokens_bf16, gate, require_gpu,
                         tokens_match)
from oracle import accept as oacc
from oracle import workload as ow
from oracle.numerics import bf16_to_f64
from vcsynth import configs as C
from vcsynth import tensors as T

pytestmark = pytest.mark.gpu


def small(name):
    base = C.get(name)
    if name == "C1":
        return base
    if name == "C2":
        return C.scaled(base, L=2, B=2, n=1000)
    if name == "C3":
        return C.scaled(base, L=2, B=2, n=1000)
    if name == "C4":
        return C.scaled(base, L=2, B=2, n=1200)
    if name == "C5":
        cfg = C.scaled(base, B=10)
        for r in cfg.reqs:  # keep the ragged mix, shrink the lengths
            r.ctx_len = max(90, r.ctx_len // 40)
            if r.comp == C.COMP_DROP:
                r.top = r.ctx_len // 4
        return cfg
    raise KeyError(name)


@functools.lru_cache(maxsize=2)
def built(name):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = small(name)
    wl = Workload(cfg)
    if cfg.mixed:
        wl.run_mixed()
    else:
        for i in range(max(r.x for r in cfg.reqs)):
            wl.run_draft(i)
        wl.run_verify()
        wl.logits_and_accept()
    torch.cuda.synchronize()
    return cfg, wl


def test_generator_gpu_matches_cpu():
    cfg, wl = built("C1")
    assert np.array_equal(wl.q[0, 0, :8].view(torch.int16).cpu().numpy().view(np.uint16),
                          T.q_bits(cfg, 0, 0, 8))
    k, v = pool_tokens_bf16(wl.full, 0, 0, 1, cfg.reqs[0].ctx_len, cfg.d)
    assert np.array_equal(k, bf16_to_f64(T.kctx_bits(cfg, 0, 0, 1, cfg.reqs[0].ctx_len)))
    assert np.array_equal(v, bf16_to_f64(T.vctx_bits(cfg, 0, 0, 1, cfg.reqs[0].ctx_len)))
    assert np.array_equal(wl.w_u.view(torch.int16).cpu().numpy().view(np.uint16), T.wu_bits(cfg))
    kb = wl.blk_k[0, 0, 1].reshape(-1, cfg.d).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(kb[:8], T.kblk_bits(cfg, 0, 0, 1, 8))
    vb = wl.blk_v[0, 0, 1].permute(0, 2, 1).reshape(-1, cfg.d).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(vb[:8], T.vblk_bits(cfg, 0, 0, 1, 8))


@pytest.mark.parametrize("name", ["C1", "C2", "C4", "C5"])
def test_kept_sets_bit_exact(name):
    cfg, wl = built(name)
    for r, req in enumerate(cfg.reqs):
        if req.comp not in (C.COMP_DROP, C.COMP_DROP_KIVI4) or req.kind == C.KIND_VERIFY:
            continue
        for l in range(cfg.L):
            for g in range(cfg.Hkv):
                want = ow.cmp.kept_positions(T.scores_u32(cfg, r, l, g, req.ctx_len), req.ctx_len,
                                             req.recent, req.top)
                got = wl.kept[r, l, g, :req.kept].cpu().numpy()
                assert np.array_equal(got, want), (r, l, g)


@pytest.mark.parametrize("name", ["C3", "C4", "C5"])
def test_kivi_codes_bit_exact(name):
    cfg, wl = built(name)
    for r, req in enumerate(cfg.reqs):
        if req.comp not in (C.COMP_KIVI2, C.COMP_DROP_KIVI4) or req.kind == C.KIND_VERIFY:
            continue
        for l in range(cfg.L):
            for g in range(cfg.Hkv):
                cm = ow.compressed(cfg, r, l, g)
                got = pool_kivi(wl.kivi_pool, l, r, g, req.kept, cfg.d)
                for key in ("kcodes", "vcodes"):
                    assert np.array_equal(got[key], getattr(cm, key)), (key, r, l, g)
                for key in ("kscale", "kzero", "vscale", "vzero"):
                    assert np.array_equal(got[key].view(np.uint16), getattr(cm, key).view(np.uint16)), (key, r, l, g)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_verify_parity(name):
    cfg, wl = built(name)
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            want, spr = ow.verify_out(cfg, r, l, spread=True)
            got = wl.out_v[r, l, :req.x].double().cpu().numpy()
            worst = max(worst, assert_close(got, want, gate(spr), f"{name} verify r={r} l={l}"))
    print(f"{name} verify max-abs error {worst:.3e}")


def wide_cfg(kind):
    """Verify launches of more than 128 query rows (x * G) per (layer, kv head)."""
    c4 = C.get("C4")
    if kind == "g8_x17":    # 136 rows = 5 blocks: 4 whole-block waves and 2 half waves
        return C.scaled(c4, L=1, B=2, n=900, x=17)
    if kind == "g8_x64":    # 512 rows: two row groups of 256 (8 waves)
        return C.scaled(c4, L=1, B=1, n=700, x=64)
    if kind == "g16_d64":   # G = 16, d = 64: 24 * 16 = 384 rows (12 waves), and a request of 3 * 16
        reqs = [C.Request(ctx_len=650, x=24, comp=C.COMP_DROP, recent=64, top=650 // 4),
                C.Request(ctx_len=333, x=3, comp=C.COMP_DROP, recent=64, top=333 // 4)]
        return C.Config("wide-g16-d64", 41, L=1, Hq=32, Hkv=2, d=64, reqs=reqs, wu_width=512,
                        vocab=1024)
    if kind == "g8_d64_x40":  # G = 8, d = 64: 40 * 8 = 320 rows = 10 blocks, the last two split by
        # key half over four waves (12 waves); the second request (24 * 8 = 192 rows) leaves the
        # split waves without rows
        reqs = [C.Request(ctx_len=777, x=40, comp=C.COMP_DROP, recent=64, top=777 // 4),
                C.Request(ctx_len=401, x=24, comp=C.COMP_DROP, recent=64, top=401 // 4)]
        return C.Config("wide-g8-d64", 42, L=2, Hq=16, Hkv=2, d=64, reqs=reqs, wu_width=1024,
                        vocab=1024)
    raise KeyError(kind)


@pytest.mark.parametrize("kind,split_pages", [("g8_x17", 0), ("g8_x17", 8), ("g8_x64", 0),
                                              ("g16_d64", 0), ("g16_d64", 4),
                                              ("g8_d64_x40", 0), ("g8_d64_x40", 8)])
def test_wide_verify_parity(kind, split_pages):
    """Every output element of the wide verify work-groups (one wave per 32 rows, 5 to 12 waves)
    against the oracle, unsplit and with context splits of 2 and 1 tiles (partials + merge)."""
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = wide_cfg(kind)
    print(f"wide verify {kind} split_pages={split_pages}", flush=True)
    wl = Workload(cfg, build_compressed=False)
    wl.run_verify(split_pages)
    torch.cuda.synchronize()
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            want, spr = ow.verify_out(cfg, r, l, spread=True)
            got = wl.out_v[r, l, :req.x].double().cpu().numpy()
            worst = max(worst, assert_close(got, want, gate(spr), f"{kind} verify r={r} l={l}"))
    print(f"{kind} verify max-abs error {worst:.3e}")


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_draft_parity(name):
    cfg, wl = built(name)
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            cc = [ow.compressed(cfg, r, l, g) for g in range(cfg.Hkv)]
            want, spr = ow.draft_out(cfg, r, l, range(req.x), comp_cache=cc, spread=True)
            got = wl.out_d[r, l, :req.x].double().cpu().numpy()
            tol = gate(spr, kivi=req.bits != 16)
            worst = max(worst, assert_close(got, want, tol, f"{name} draft r={r} l={l}"))
    print(f"{name} draft max-abs error {worst:.3e}")


def test_mixed_ragged_parity():
    cfg, wl = built("C5")
    for r, req in enumerate(cfg.reqs):
        if req.kind == C.KIND_VERIFY:
            want, spr = ow.verify_out(cfg, r, 0, spread=True)
            got = wl.out_v[r, 0, :req.x].double().cpu().numpy()
            assert_close(got, want, gate(spr), f"C5 verify r={r}")
        else:
            want, spr = ow.draft_out(cfg, r, 0, [req.step], spread=True)
            want, spr = want[0], spr[0]
            got = wl.out_v[r, 0, req.step].double().cpu().numpy()
            assert_close(got, want, gate(spr, kivi=req.bits != 16),
                         f"C5 draft r={r} ({req.comp}, step {req.step})")


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_tokens_and_accept(name):
    cfg, wl = built(name)
    tok_d = wl.tok_d.cpu().numpy()
    tok_v = wl.tok_v.cpu().numpy()
    alen = wl.acc_len.cpu().numpy()
    nxt = wl.next_tok.cpu().numpy()
    zd = wl.z_d.cpu().numpy().reshape(cfg.B * cfg.L, wl.xmax, -1)
    zv = wl.z_v.cpu().numpy().reshape(cfg.B * cfg.L, wl.xmax, -1)
    flagged = 0
    for r, req in enumerate(cfg.reqs):
        x = req.x
        for l in range(cfg.L):
            inst = r * cfg.L + l
            res = ow.round_instance(cfg, r, l)
            assert not tokens_match(tok_d[inst, :x], res.draft_tok, res.draft_gap, res.draft_logits)
            assert not tokens_match(tok_v[inst, :x], res.verify_tok, res.verify_gap, res.verify_logits)
            if res.flagged:
                flagged += 1
            else:
                assert alen[inst] == res.accept_len and nxt[inst] == res.next_tok
            # the accept kernel itself, on the GPU's own logits, is exact
            td, _ = oacc.argmax_gap(zd[inst, :x].astype(np.float64))
            tv, _ = oacc.argmax_gap(zv[inst, :x].astype(np.float64))
            assert np.array_equal(tok_d[inst, :x], td) and np.array_equal(tok_v[inst, :x], tv)
            assert (alen[inst], nxt[inst]) == oacc.accept(td, tv)
    print(f"{name}: {flagged} flagged accept lengths of {cfg.B * cfg.L}")


def test_mixed_ragged_tokens():
    """Tokens of the ragged mixed launch: the LM-head stand-in and the accept kernel's argmax over
    every verify row of the verifying requests and the draft-step row of the drafting ones,
    against the oracle's tokens (flagged near-ties excepted)."""
    cfg, wl = built("C5")
    wl.logits_and_accept()
    torch.cuda.synchronize()
    tok = wl.tok_v.cpu().numpy().reshape(cfg.B, wl.xmax)
    wu = bf16_to_f64(T.wu_bits(cfg))
    checked = 0
    for r, req in enumerate(cfg.reqs):
        if req.kind == C.KIND_VERIFY:
            rows, o = list(range(req.x)), ow.verify_out(cfg, r, 0)
        else:
            rows, o = [req.step], ow.draft_out(cfg, r, 0, [req.step])
        z = oacc.logits(o.reshape(len(rows), -1), wu)
        t, gap = oacc.argmax_gap(z)
        assert not tokens_match(tok[r, rows], t, gap, z), f"C5 tokens r={r}"
        checked += len(rows)
    print(f"C5: {checked} token rows checked")
