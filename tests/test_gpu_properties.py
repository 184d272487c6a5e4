"""Properties the method fixes, checked on the GPU path against the oracle (run on an MI355X: -m gpu).

* Lossless drafting (VeriCache review, §Draft–Verify Pipeline: the drafter is lossy only through
  its key set and values): a drafting cache that keeps every context token gives draft step i
  the key set and values of verify row i.  The draft and verify kernels then agree to their own
  rounding, their argmax tokens agree except at near-ties the oracle flags, and every drafted
  token is accepted (a = x).
* Verify with one drafted row is a decode step: it equals draft step 0 over the same keep-all
  cache.
* A request with no context tokens attends only to its drafted block (rows 0..i), in both passes.
* KIVI quantisation that is exact on its inputs (context values on the quantiser's lattice) makes
  the 2- and 4-bit drafters lossless too: the KIVI draft kernel matches the verify kernel.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, gate, require_gpu, tokens_match
from oracle import attention as oatt
from oracle import workload as ow
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def keep_all(cfg):
    for r in cfg.reqs:
        r.comp, r.recent, r.top = C.COMP_DROP, r.ctx_len, 0
    return cfg


def run_round(cfg):
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    wl = Workload(cfg)
    for i in range(max(r.x for r in cfg.reqs)):
        wl.run_draft(i)
    wl.run_verify()
    wl.logits_and_accept()
    torch.cuda.synchronize()
    return wl


def outputs(wl, cfg):
    """(draft, verify) outputs as float64 [B][L][xmax][Hq][d]."""
    return (wl.out_d.cpu().numpy().astype(np.float64), wl.out_v.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name,kw", [("C1", dict(n=1000)), ("C2", dict(L=2, B=2, n=1000, x=8))])
def test_keep_all_draft_equals_verify_and_accepts_all(name, kw):
    cfg = keep_all(C.scaled(C.get(name), **kw))
    print(f"keep-all {cfg.name} {kw}", flush=True)
    wl = run_round(cfg)
    od, ov = outputs(wl, cfg)
    tok_d, tok_v = wl.tok_d.cpu().numpy(), wl.tok_v.cpu().numpy()
    alen, nxt = wl.acc_len.cpu().numpy(), wl.next_tok.cpu().numpy()
    worst = 0.0
    for r, req in enumerate(cfg.reqs):
        x = req.x
        for l in range(cfg.L):
            inst = r * cfg.L + l
            res = ow.round_instance(cfg, r, l, spread=True)
            tol_v, tol_d = gate(res.verify_spread), gate(res.draft_spread)
            # the two kernels compute the same attention: each is within its gate of the exact
            # value, so they are within the sum of the gates of each other
            worst = max(worst, assert_close(od[r, l, :x], ov[r, l, :x], tol_v + tol_d,
                                            f"draft-vs-verify r={r} l={l}"))
            assert res.accept_len == x and res.next_tok == -1  # the oracle: lossless, all accepted
            assert_close(od[r, l, :x], res.draft_o, tol_d, f"draft r={r} l={l}")
            assert_close(ov[r, l, :x], res.verify_o, tol_v, f"verify r={r} l={l}")
            assert not tokens_match(tok_d[inst, :x], res.draft_tok, res.draft_gap, res.draft_logits)
            assert not tokens_match(tok_v[inst, :x], res.verify_tok, res.verify_gap, res.verify_logits)
            if not res.flagged:
                assert np.array_equal(tok_d[inst, :x], tok_v[inst, :x])
                assert alen[inst] == x and nxt[inst] == -1
    print(f"{cfg.name}: draft-vs-verify max-abs {worst:.3e}")


def test_verify_of_one_row_is_a_decode_step():
    cfg = keep_all(C.scaled(C.get("C2"), L=2, B=2, n=777, x=1))
    print(f"x=1 {cfg.name}", flush=True)
    wl = run_round(cfg)
    od, ov = outputs(wl, cfg)
    for r, req in enumerate(cfg.reqs):
        for l in range(cfg.L):
            res = ow.round_instance(cfg, r, l, spread=True)
            tol_v, tol_d = gate(res.verify_spread), gate(res.draft_spread)
            assert_close(ov[r, l, :1], od[r, l, :1], tol_v + tol_d, f"x=1 r={r} l={l}")
            assert_close(ov[r, l, :1], res.verify_o, tol_v, f"x=1 verify r={r} l={l}")


def test_request_without_context_sees_only_its_block():
    cfg = C.scaled(C.get("C2"), L=1, B=3, n=1000, x=8)
    for r, n in zip(cfg.reqs, (1000, 0, 37)):
        r.ctx_len, r.recent, r.top = n, min(128, n), n // 4
    print(f"context lengths 1000, 0, 37 {cfg.name}", flush=True)
    wl = run_round(cfg)
    od, ov = outputs(wl, cfg)
    for r, req in enumerate(cfg.reqs):
        x = req.x
        res = ow.round_instance(cfg, r, 0, spread=True)
        tol_v, tol_d = gate(res.verify_spread), gate(res.draft_spread)
        assert_close(ov[r, 0, :x], res.verify_o, tol_v, f"verify n={req.ctx_len}")
        assert_close(od[r, 0, :x], res.draft_o, tol_d, f"draft n={req.ctx_len}")
        if req.ctx_len == 0:
            # nothing but the drafted block, in both passes: the same keys, so the same outputs
            assert_close(od[r, 0, :x], ov[r, 0, :x], tol_v + tol_d, "n=0 draft-vs-verify")


def lattice_context(n, d, hkv, bits, seed):
    """Context K or V [1][hkv][n][d] on the KIVI lattice z + s*code with s = 4 / (Lq + 1) and
    z = -Lq*s/2 (2-bit: -1.5, -0.5, 0.5, 1.5; 4-bit: -1.875 .. 1.875 in steps of 1/4; exact in
    bf16 and fp16).  Code 0 sits where (token - channel) % 32 == 0 and Lq where it is 1, so every
    32-token key group of a channel and every 32-channel value group of a token holds both ends:
    its min-max quantisation recovers s, z and the codes exactly.  Other codes are seeded draws."""
    lq = (1 << bits) - 1
    gen = torch.Generator().manual_seed(seed)
    codes = torch.randint(0, lq + 1, (1, hkv, n, d), generator=gen)
    diff = (torch.arange(n).view(n, 1) - torch.arange(d).view(1, d)) % 32
    codes[:, :, diff == 0] = 0
    codes[:, :, diff == 1] = lq
    step = 4.0 / (lq + 1)
    return (-lq * step / 2 + step * codes.double()).to(torch.bfloat16)


@pytest.mark.parametrize("comp,bits,base", [(C.COMP_KIVI2, 2, "C3"), (C.COMP_DROP_KIVI4, 4, "C4")])
def test_lattice_kivi_draft_equals_verify_and_accepts_all(comp, bits, base):
    """Quantisation that is exact on its inputs makes the KIVI drafter lossless: the KIVI draft
    kernel and the verify kernel see the same keys and values, so they agree to their rounding and
    every drafted token is accepted.  Rows whose verify top-2 logit gap is under 1e-3 are near-ties
    (flagged, as in the oracle comparisons): tokens are compared on the other rows, and the accept
    length must reach the first near-tie row."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    from lossless_kv_cache_vc_amd.harness import Workload
    cfg = C.scaled(C.get(base), L=2, B=2, n=1024, x=8)
    for r in cfg.reqs:
        r.comp, r.recent, r.top = comp, r.ctx_len, 0   # drop + KIVI-4: keep every token
    print(f"lattice KIVI-{bits} {cfg.name}", flush=True)
    wl = Workload(cfg, build_compressed=False)
    lat = {}
    for r, n in enumerate(wl.lens):
        row = wl._row(wl.full, r)
        for l in range(cfg.L):
            for which in (0, 1):
                lat[(r, l, which)] = lattice_context(n, cfg.d, cfg.Hkv, bits, seed=1000 * r + 10 * l + which)
                src = lat[(r, l, which)].to(wl.dev)
                vc.pack_bf16(wl.shape, [n], l, src, n, row, which)
    wl._build_compressed(False)
    wl.workspace = wl._workspace()
    for i in range(max(r.x for r in cfg.reqs)):
        wl.run_draft(i)
    wl.run_verify()
    wl.logits_and_accept()
    torch.cuda.synchronize()
    od, ov = outputs(wl, cfg)
    tok_d, tok_v = wl.tok_d.cpu().numpy(), wl.tok_v.cpu().numpy()
    alen = wl.acc_len.cpu().numpy()
    zv = wl.z_v.cpu().numpy().reshape(cfg.B * cfg.L, wl.xmax, -1)
    worst, full = 0.0, 0
    for r, req in enumerate(cfg.reqs):
        x = req.x
        for l in range(cfg.L):
            inst = r * cfg.L + l
            # each pass within its gate of the exact attention over the lattice context
            q, G = ow.queries(cfg, r, l, x), cfg.G
            spr = np.concatenate([oatt.verify_unit(q[:, g * G:(g + 1) * G],
                                                   lat[(r, l, 0)][0, g].double().numpy(),
                                                   lat[(r, l, 1)][0, g].double().numpy(),
                                                   *ow.block(cfg, r, l, g, x), spread=True)[1]
                                  for g in range(cfg.Hkv)], axis=1)
            worst = max(worst, assert_close(od[r, l, :x], ov[r, l, :x], gate(spr) + gate(spr, kivi=True),
                                            f"KIVI-{bits} draft-vs-verify r={r} l={l}"))
            top2 = np.sort(zv[inst, :x], axis=1)[:, -2:]
            clear = (top2[:, 1] - top2[:, 0]) >= 1e-3
            assert np.array_equal(tok_d[inst, :x][clear], tok_v[inst, :x][clear])
            # accepted at least up to the first near-tie row (all x when there is none)
            first = int(np.argmin(clear)) if not clear.all() else x
            assert alen[inst] >= first
            full += first == x
    print(f"KIVI-{bits}: draft-vs-verify max-abs {worst:.3e}; {full} of {cfg.B * cfg.L} instances "
          f"without a near-tie row, all accepted")
