"""Rejection-sampling accept and drafter sampling on the GPU against the float64 oracle
(VeriCache review, §Implementation notes, "Rejection sampling for non-greedy").

Tokens and accept decisions are integers decided by float64 comparisons on both sides; they must
be equal except where the oracle flags a decision within 1e-9 (relative) of its threshold, where
another summation order may take the other side."""
import numpy as np
import pytest
import torch

from gpu_helpers import require_gpu
from oracle import sampling as S
from vcsynth import rng

pytestmark = pytest.mark.gpu

SEED = 0x5EED0100


def _normals(stream, n, salt=0):
    # N(0, 1) from the seeded generator (Box-Muller on two uniforms), as float32
    i = np.arange(n, dtype=np.int64) + (salt << 40)
    u1 = rng.uniform01(SEED, stream, 2 * i)
    u2 = rng.uniform01(SEED, stream, 2 * i + 1)
    return (np.sqrt(-2 * np.log(u1)) * np.cos(2 * np.pi * u2)).astype(np.float32)


def _uniforms(stream, n, salt=0):
    return rng.uniform01(SEED, stream, np.arange(n, dtype=np.int64) + (salt << 40))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(n_inst, max_x, V, T, salt, drift=0.3, scale=2.0):
    """Verifier logits N(0, scale^2), drafter logits = verifier + drift * N(0, 1) (fp32)."""
    zv = scale * _normals(rng.STREAM_Q, n_inst * (max_x + 1) * V, salt).reshape(n_inst, max_x + 1, V)
    zd = zv[:, :max_x] + np.float32(drift) * _normals(rng.STREAM_KBLK, n_inst * max_x * V, salt).reshape(n_inst, max_x, V)
    return zd.astype(np.float32), zv.astype(np.float32)


def _run(zd, zv, x, xv, T, salt, draft_tok=None):
    from lossless_kv_cache_vc_amd import vc
    n_inst, max_x, V = zd.shape
    max_xv = zv.shape[1]
    T32 = float(np.float32(T))  # the library takes fp32 T; the oracle uses that exact value
    ud = _uniforms(rng.STREAM_UDRAFT, n_inst * max_x, salt)
    ua = _uniforms(rng.STREAM_UACC, n_inst * max_x, salt).reshape(n_inst, max_x)
    ur = _uniforms(rng.STREAM_URES, n_inst * (max_x + 1), salt).reshape(n_inst, max_x + 1)
    zd_d, zv_d = _dev(zd), _dev(zv)
    tok_d = torch.empty(n_inst * max_x, dtype=torch.int32, device="cuda")
    vc.sample_tokens(n_inst * max_x, V, T32, zd_d, _dev(ud), tok_d)
    if draft_tok is not None:
        tok_d = _dev(draft_tok.astype(np.int32).reshape(-1))
    alen = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    nxt = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    vc.accept_sampled(n_inst, max_x, max_xv, V, T32, _dev(x.astype(np.int32)), _dev(xv.astype(np.int32)),
                      zd_d, zv_d, tok_d, _dev(ua), _dev(ur), alen, nxt)
    torch.cuda.synchronize()
    return T32, ud, ua, ur, tok_d.cpu().numpy().reshape(n_inst, max_x), alen.cpu().numpy(), nxt.cpu().numpy()


def _check(zd, zv, x, xv, T, salt, draft_tok=None, check_sampling=True):
    T32, ud, ua, ur, gtok, galen, gnxt = _run(zd, zv, x, xv, T, salt, draft_tok)
    n_inst, max_x, V = zd.shape
    print(f"sampled accept: {n_inst} instances, x <= {max_x}, vocab {V}, T = {T}", flush=True)
    if check_sampling and draft_tok is None:
        otok, oflag = S.sample_tokens(zd.reshape(-1, V), T32, ud)
        mism = (otok != gtok.reshape(-1)) & ~oflag
        assert not mism.any(), f"drafter sampling differs at rows {np.nonzero(mism)[0][:8]}"
    stats = {"flagged": 0, "accepted": 0}
    for i in range(n_inst):
        nx, nxv = int(x[i]), int(xv[i])
        a, nxt, flag = S.accept_sampled(zd[i, :nx], zv[i, :nxv], gtok[i, :nx], T32, ua[i, :nx], ur[i, :nx + 1])
        if flag:
            stats["flagged"] += 1
            continue
        assert (int(galen[i]), int(gnxt[i])) == (a, nxt), f"instance {i}: gpu {(galen[i], gnxt[i])}, oracle {(a, nxt)}"
        stats["accepted"] += a
    return stats


@pytest.mark.parametrize("T", [1.0, 0.7, 0.3])
def test_sampled_accept_full_round_count(T):
    """The Llama-3.1-8B 32K round's 256 instances (8 requests x 32 layer slices), 32 slots,
    vocabulary 4096; mixed block lengths, half with a bonus row."""
    require_gpu()
    n_inst, max_x, V = 256, 32, 4096
    zd, zv = _case(n_inst, max_x, V, T, salt=int(T * 10))
    u = _uniforms(rng.STREAM_DRAWS, n_inst, salt=int(T * 10))
    x = np.where(np.arange(n_inst) % 4 == 3, 1 + (u * max_x).astype(np.int64) % max_x, max_x)
    xv = x + (np.arange(n_inst) % 2)
    st = _check(zd, zv, x, xv, T, salt=int(T * 10))
    assert st["flagged"] <= 2
    # the drift makes rejections common but not universal
    assert 0 < st["accepted"] < x.sum()


def test_identical_caches_keep_every_slot():
    require_gpu()
    n_inst, max_x, V = 32, 16, 1000
    zd, zv = _case(n_inst, max_x, V, 0.8, salt=3, drift=0.0)
    x = np.full(n_inst, max_x)
    xv = x + 1
    T32, *_rest, galen, gnxt = _run(zd, zv, x, xv, 0.8, salt=3)
    assert (galen == max_x).all()
    _check(zd, zv, x, xv, 0.8, salt=3)


def test_out_of_range_token_and_short_verifier():
    """A drafted token outside the vocabulary is never kept; xv = x gives no bonus; tiny and
    ragged vocabularies (fewer entries than threads, not a multiple of them)."""
    require_gpu()
    for V in (3, 257, 1000):
        n_inst, max_x = 8, 5
        zd, zv = _case(n_inst, max_x, V, 1.0, salt=V, drift=0.0)
        x = np.full(n_inst, max_x)
        toks = np.zeros((n_inst, max_x), dtype=np.int64)
        toks[:, 2] = V            # out of range at slot 2
        toks[0, 0] = -1           # and at slot 0 of instance 0
        T32, _, _, _, _, galen, gnxt = _run(zd, zv[:, :max_x].copy(), x, x, 1.0, salt=V, draft_tok=toks)
        assert galen[0] == 0 and (galen[1:] <= 2).all()
        assert ((gnxt >= 0) & (gnxt < V)).all()


def test_round_logits_of_the_attention_path():
    """Logits of the draft and verify passes of the 32K workload (two layer slices): drafter and
    verifier distributions are close, so most slots are kept."""
    require_gpu()
    from lossless_kv_cache_vc_amd.harness import Workload
    from vcsynth import configs as C
    cfg = C.scaled(C.get("C2"), L=2)
    wl = Workload(cfg)
    wl.run_round()
    torch.cuda.synchronize()
    n_inst, xm, V = cfg.B * cfg.L, wl.xmax, cfg.vocab
    zd = wl.z_d.view(n_inst, xm, V).cpu().numpy()
    zv = wl.z_v.view(n_inst, xm, V).cpu().numpy()
    x = np.array([cfg.reqs[i // cfg.L].x for i in range(n_inst)])
    st = _check(zd, zv, x, x.copy(), 0.7, salt=11)
    print(f"round logits: {st['accepted']} of {x.sum()} drafted slots kept, {st['flagged']} flagged", flush=True)
    assert st["flagged"] <= 1
