"""The LM-head stand-in (vc_logits) against the oracle's fp64 logits (run on an MI355X: -m gpu).

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
    (200, 256, 256, 384),     # 16-byte loads, 2 x 3 tiles with ragged rows
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
