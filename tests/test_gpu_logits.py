"""The LM-head stand-in (vc_logits) and the greedy accept (vc_accept) against the oracle (run on an
MI355X: -m gpu).

z = o * W_u with o fp32 and W_u bf16.  The kernel splits each element of o into two bf16 parts
and accumulates both products in fp32, so z differs from the exact product by the split's
residue (at most 2^-18 of each element) and fp32 accumulation; the bound checked is
2e-5 * sum_k |o_k| |W_kv| + 1e-7, elementwise.  Shapes cover the 16-byte-load path and the
scalar path (vocab not a multiple of 8, width not a multiple of 32), a row stride wider than the
width, and tiles cut by the edges of rows and vocab.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import require_gpu
from oracle import accept as oacc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,width,ld_o,vocab", [
    (200, 256, 256, 384),     # 16-byte loads, 2 x 2 tiles (128 x 256), ragged rows and vocabulary
    (130, 64, 72, 136),       # 16-byte loads, row stride > width
    (75, 100, 104, 203),      # scalar loads: vocab % 8 != 0, width % 32 != 0
    (1, 4096, 4096, 4096),    # one row at the 8B shape's width and vocabulary
])
def test_logits_match_the_oracle(rows, width, ld_o, vocab):
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    print(f"logits rows={rows} width={width} ld_o={ld_o} vocab={vocab}", flush=True)
    g = torch.Generator().manual_seed(rows * 7 + width)
    o = torch.randn((rows, ld_o), generator=g, dtype=torch.float32)
    w = (torch.randn((width, vocab), generator=g, dtype=torch.float32) / np.sqrt(width)).to(torch.bfloat16)
    z = torch.full((rows, vocab), float("nan"), dtype=torch.float32, device="cuda")
    o_d, w_d = o.cuda(), w.cuda()
    vc.logits(rows, width, vocab, o_d, ld_o, w_d, z)
    torch.cuda.synchronize()
    got = z.cpu().numpy().astype(np.float64)
    o64 = o[:, :width].numpy().astype(np.float64)
    w64 = w.float().numpy().astype(np.float64)
    want = oacc.logits(o64, w64)
    bound = 2e-5 * (np.abs(o64) @ np.abs(w64)) + 1e-7
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max error {err.max():.3e}, worst ratio {(err / bound).max():.2f}"
    print(f"max abs error {err.max():.3e} (bound at that element {bound.flat[err.argmax()]:.3e})")


@pytest.mark.parametrize("vocab", [4096, 1001, 37])
def test_greedy_accept_matches_the_oracle(vocab):
    """vc_accept on random logits with planted exact ties (the lowest index must win) and planted
    agreement, for the 16-byte-load path (vocab % 4 == 0) and the scalar one; block lengths 1..64,
    half of them with a bonus verifier row (xv = x + 1).  Tokens, accept lengths and next tokens
    must equal the oracle's exactly."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    print(f"greedy accept vocab={vocab}", flush=True)
    rng = np.random.default_rng(vocab)
    n_inst, max_x = 48, 64
    max_xv = max_x + 1
    x = rng.integers(1, max_x + 1, n_inst).astype(np.int32)
    xv = (x + (np.arange(n_inst) % 2)).astype(np.int32)
    zd = rng.standard_normal((n_inst, max_x, vocab)).astype(np.float32)
    zv = rng.standard_normal((n_inst, max_xv, vocab)).astype(np.float32)
    for i in range(n_inst):
        agree = rng.integers(0, x[i] + 1)  # rows before `agree` share their argmax
        for j in range(x[i]):
            t = rng.integers(0, vocab)
            if j < agree:
                zd[i, j, t] = zv[i, j, t] = 10.0
            if j % 3 == 0:  # an exact tie: the lower index must win
                u = rng.integers(0, vocab)
                zd[i, j, u] = zd[i, j].max()
                zv[i, j, u] = zv[i, j].max()
    to = lambda a: torch.from_numpy(a).cuda()
    dt = torch.empty((n_inst, max_x), dtype=torch.int32, device="cuda")
    vt = torch.empty((n_inst, max_xv), dtype=torch.int32, device="cuda")
    al = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    nt = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    vc.accept(n_inst, max_x, max_xv, vocab, to(x), to(xv), to(zd), to(zv), dt, vt, al, nt)
    torch.cuda.synchronize()
    dt, vt, al, nt = dt.cpu().numpy(), vt.cpu().numpy(), al.cpu().numpy(), nt.cpu().numpy()
    for i in range(n_inst):
        td, _ = oacc.argmax_gap(zd[i, :x[i]].astype(np.float64))
        tv, _ = oacc.argmax_gap(zv[i, :xv[i]].astype(np.float64))
        assert np.array_equal(dt[i, :x[i]], td) and np.all(dt[i, x[i]:] == -1)
        assert np.array_equal(vt[i, :xv[i]], tv) and np.all(vt[i, xv[i]:] == -1)
        assert (al[i], nt[i]) == oacc.accept(td, tv)


@pytest.mark.parametrize("max_x,max_xv", [(64, 65), (40, 24)])
def test_greedy_accept_short_verifier(max_x, max_xv):
    """Instances whose verifier has fewer rows than drafted slots (xv < x), including a launch with
    max_xv < max_x: only slots with a verifier row are compared, so accept_len <= xv and next_tok is
    -1 when every compared slot agrees.  The logits rows past each instance's xv are NaN-free noise
    with an agreeing argmax planted, so a kernel that read past xv would return a longer block."""
    require_gpu()
    from lossless_kv_cache_vc_amd import vc
    print(f"greedy accept short verifier max_x={max_x} max_xv={max_xv}", flush=True)
    rng = np.random.default_rng(max_x * 100 + max_xv)
    n_inst, vocab = 40, 512
    x = rng.integers(1, max_x + 1, n_inst).astype(np.int32)
    # verifier rows: at most x + 1 (the bonus row), here mostly fewer than x
    xv = np.minimum(np.minimum(rng.integers(0, max_x + 1, n_inst), x + 1), max_xv).astype(np.int32)
    xv[:4] = np.minimum([0, 1, x[2] - 1, x[3] + 1], max_xv).clip(0)
    zd = rng.standard_normal((n_inst, max_x, vocab)).astype(np.float32)
    zv = rng.standard_normal((n_inst, max_xv, vocab)).astype(np.float32)
    for i in range(n_inst):
        agree = rng.integers(0, max_x + 1)   # drafted slots before `agree` match the verifier's rows
        for j in range(min(agree, max_xv)):
            t = rng.integers(0, vocab)
            zd[i, j, t] = zv[i, j, t] = 10.0
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dt = torch.empty((n_inst, max_x), dtype=torch.int32, device="cuda")
    vt = torch.empty((n_inst, max_xv), dtype=torch.int32, device="cuda")
    al = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    nt = torch.empty(n_inst, dtype=torch.int32, device="cuda")
    for rep in range(2):   # the second launch, with the verifier lengths permuted, must not see
        if rep:            # the first one's tokens
            xv = np.minimum(np.minimum(xv[::-1], x + 1), max_xv).astype(np.int32)
        vc.accept(n_inst, max_x, max_xv, vocab, to(x), to(xv), to(zd), to(zv), dt, vt, al, nt)
        torch.cuda.synchronize()
        d_, v_, a_, n_ = dt.cpu().numpy(), vt.cpu().numpy(), al.cpu().numpy(), nt.cpu().numpy()
        for i in range(n_inst):
            td, _ = oacc.argmax_gap(zd[i, :x[i]].astype(np.float64))
            tv, _ = oacc.argmax_gap(zv[i, :xv[i]].astype(np.float64)) if xv[i] else (np.zeros(0, np.int64), None)
            assert np.array_equal(d_[i, :x[i]], td)
            assert np.array_equal(v_[i, :xv[i]], tv) and np.all(v_[i, xv[i]:] == -1)
            assert (a_[i], n_[i]) == oacc.accept_block(td, tv), (i, x[i], xv[i])
            assert a_[i] <= min(x[i], xv[i])
