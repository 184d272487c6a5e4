"""Committing accepted rows (VeriCache review, §Draft–Verify Pipeline, per-request cycle: accepted
positions join the caches, rejected ones are rolled back) against the oracle.

After a commit of c_r block rows per request, the full cache must hold the context followed by
block rows 0..c_r-1; the token-drop cache must hold the full cache at the old kept positions
followed by the new positions (new tokens are always kept); a KIVI cache must hold the
quantisation of the grown storage sequence, bit for bit (a key group that gained tokens is
re-quantised).  The next round's draft and verify attention over the grown caches must match the
oracle.  Rows from c_r on are never written (the rollback)."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, pool_kivi, pool_tokens_bf16, gate, require_gpu
from oracle import attention as oatt
from oracle import compress as ocmp
from oracle import workload as ow
from oracle.numerics import bf16_to_f64
from vcsynth import configs as C
from vcsynth import tensors as T

pytestmark = pytest.mark.gpu

# n = 316 puts the full and KIVI-2 tails 28 tokens into a 32-token group, so a commit of 8 rows
# crosses both a page and a key-group boundary; the drop caches keep 128 + 79 = 207 tokens.
COUNTS = [8, 3]


def _cfg(name):
    return C.scaled(C.get(name), L=2, B=2, n=316, x=8)


def _grown(cfg, r, l, g, c):
    """Full context of (r, l, g) after committing c block rows: (k, v) float64 [n + c][d]."""
    n = cfg.reqs[r].ctx_len
    x = cfg.reqs[r].x
    k = np.concatenate([bf16_to_f64(T.kctx_bits(cfg, r, l, g, n)), bf16_to_f64(T.kblk_bits(cfg, r, l, g, x))[:c]])
    v = np.concatenate([bf16_to_f64(T.vctx_bits(cfg, r, l, g, n)), bf16_to_f64(T.vblk_bits(cfg, r, l, g, x))[:c]])
    return k, v


def _kept(cfg, r, l, g, c):
    req = cfg.reqs[r]
    n = req.ctx_len
    base = ocmp.kept_positions(T.scores_u32(cfg, r, l, g, n), n, req.recent, req.top)
    return np.concatenate([base, np.arange(n, n + c)])


def _comp(cfg, r, l, g, c):
    """The grown drafting cache: ow.Compressed over the grown storage sequence."""
    req = cfg.reqs[r]
    k, v = _grown(cfg, r, l, g, c)
    kept = _kept(cfg, r, l, g, c) if req.comp in (C.COMP_DROP, C.COMP_DROP_KIVI4) else None
    ks, vs = (k[kept], v[kept]) if kept is not None else (k, v)
    if req.comp == C.COMP_DROP:
        return ow.Compressed(k=ks, v=vs, kept=kept)
    kc, ksc, kz = ocmp.quantize_keys(ks, req.bits)
    vc, vsc, vz = ocmp.quantize_values(vs, req.bits)
    return ow.Compressed(k=ocmp.dequantize_keys(kc, ksc, kz), v=ocmp.dequantize_values(vc, vsc, vz),
                         kept=kept, kcodes=kc, kscale=ksc, kzero=kz, vcodes=vc, vscale=vsc, vzero=vz)


@pytest.fixture(scope="module", params=["C2", "C3", "C4"])
def committed(request):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = _cfg(request.param)
    print(f"commit: {cfg.name}, n = 316, counts {COUNTS}", flush=True)
    wl = Workload(cfg, spare_tokens=64)
    wl.run_round()
    free0 = {k: a.free_count(0) for k, (_, a, _) in wl._grow.items()}
    old = (list(wl.lens), list(wl.comp_lens))
    wl.commit(COUNTS)
    torch.cuda.synchronize()
    return cfg, wl, old, free0


def test_caches_after_commit(committed):
    cfg, wl, (lens0, comp0), free0 = committed
    d = cfg.d
    for r, c in enumerate(COUNTS):
        assert wl.lens[r] == lens0[r] + c and wl.comp_lens[r] == comp0[r] + c
        req = cfg.reqs[r]
        for l in range(cfg.L):
            for g in range(cfg.Hkv):
                k, v = _grown(cfg, r, l, g, c)
                gk, gv = pool_tokens_bf16(wl.full, l, r, g, wl.lens[r], d)
                assert np.array_equal(gk, k) and np.array_equal(gv, v), ("full", r, l, g)
                cm = _comp(cfg, r, l, g, c)
                if cm.kept is not None:
                    got = wl.kept[r, l, g, :wl.comp_lens[r]].cpu().numpy()
                    assert np.array_equal(got, cm.kept), ("kept", r, l, g)
                if req.comp == C.COMP_DROP:
                    dk, dv = pool_tokens_bf16(wl.drop_pool, l, r, g, wl.comp_lens[r], d)
                    assert np.array_equal(dk, cm.k) and np.array_equal(dv, cm.v), ("drop", r, l, g)
                else:
                    got = pool_kivi(wl.kivi_pool, l, r, g, wl.comp_lens[r], d)
                    for key in ("kcodes", "vcodes"):
                        assert np.array_equal(got[key], getattr(cm, key)), (key, r, l, g)
                    for key in ("kscale", "kzero", "vscale", "vzero"):
                        assert np.array_equal(got[key].view(np.uint16), getattr(cm, key).view(np.uint16)), (key, r, l, g)
    # the page allocator handed out exactly the pages the growth needed
    for name, (_, alloc, _) in wl._grow.items():
        if name == "full":
            need = sum((lens0[r] + c + 15) // 16 - (lens0[r] + 15) // 16 for r, c in enumerate(COUNTS))
        else:
            need = sum((comp0[r] + c + 15) // 16 - (comp0[r] + 15) // 16 for r, c in enumerate(COUNTS))
        assert free0[name] - alloc.free_count(0) == need, name


def test_next_round_over_grown_caches(committed):
    cfg, wl, _, _ = committed
    wl.out_v.zero_()
    wl.out_d.zero_()
    wl.run_verify()
    x = cfg.reqs[0].x
    for i in range(x):
        wl.run_draft(i)
    torch.cuda.synchronize()
    G = cfg.G
    worst_v = worst_d = 0.0
    for r, c in enumerate(COUNTS):
        req = cfg.reqs[r]
        for l in range(cfg.L):
            q = ow.queries(cfg, r, l, x)
            for g in range(cfg.Hkv):
                k, v = _grown(cfg, r, l, g, c)
                kb, vb = ow.block(cfg, r, l, g, x)
                sl = slice(g * G, (g + 1) * G)
                want, spr = oatt.verify_unit(q[:, sl], k, v, kb, vb, spread=True)
                got = wl.out_v[r, l, :x, sl].double().cpu().numpy()
                worst_v = max(worst_v, assert_close(got, want, gate(spr), f"{cfg.name} verify r={r} l={l} g={g}"))
                cm = _comp(cfg, r, l, g, c)
                res = [oatt.draft_unit(q[i, sl], cm.k, cm.v, kb, vb, i, spread=True) for i in range(x)]
                want, spr = np.stack([a for a, _ in res]), np.stack([b for _, b in res])
                got = wl.out_d[r, l, :x, sl].double().cpu().numpy()
                worst_d = max(worst_d, assert_close(got, want, gate(spr, kivi=req.bits != 16),
                                                    f"{cfg.name} draft r={r} l={l} g={g}"))
    print(f"{cfg.name} after commit: verify {worst_v:.2e}, draft {worst_d:.2e}", flush=True)


def test_zero_count_commit_changes_nothing(committed):
    cfg, wl, _, _ = committed
    # bitwise: blocks no request has written yet hold whatever the allocator left (NaN patterns
    # included), so a float comparison could fail where no bit changed
    before = (list(wl.lens), list(wl.comp_lens), wl.full.k.view(torch.int16).clone())
    wl.commit([0] * cfg.B)
    torch.cuda.synchronize()
    assert wl.lens == before[0] and wl.comp_lens == before[1]
    assert torch.equal(wl.full.k.view(torch.int16), before[2])
