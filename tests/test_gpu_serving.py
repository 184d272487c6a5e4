"""The one-GPU serving loop (VeriCache review, §KV Swap Scheduling and §Runtime Algorithm Deep
Dive, "Execution loop"): with reloads staggered by the library's Admit scheduler, or in lock-step,
every verify reads a full cache staged from pinned host memory; its output must equal the verify
over the resident cache bit for bit, and every request must keep verifying."""
import pytest
import torch

from gpu_helpers import require_gpu
from vcsynth import configs as C

pytestmark = pytest.mark.gpu


def test_staged_verifies_equal_resident_ones():
    require_gpu()
    from lossless_kv_cache_vc_amd.serving import ServeLoop
    cfg = C.scaled(C.get("C2"), L=4, B=4, n=1500, x=8)
    loop = ServeLoop(cfg)
    B, x = cfg.B, loop.x
    ref = {}
    for r in range(B):
        out = torch.zeros_like(loop.wl.out_v)
        loop.verify(r, loop.full_k[r], loop.full_v[r], out)
        ref[r] = out[r].clone()
    torch.cuda.synchronize()
    t_iter, bw = loop.measure(reps=2)
    print(f"serving loop: draft iteration {t_iter * 1e3:.3f} ms, link {bw / 1e9:.1f} GB/s", flush=True)

    # staggered: check each verify right after it runs
    seen = {r: 0 for r in range(B)}
    orig = loop.verify

    def checked(r, k, v, out=None):
        buf = torch.zeros_like(loop.wl.out_v)
        orig(r, k, v, buf)
        torch.cuda.synchronize()
        assert torch.equal(buf[r], ref[r]), f"staged verify of request {r} differs"
        seen[r] += 1
    loop.verify = checked
    # long enough for every request to be reloaded once: reloads are serial on the link
    import math
    span = max(1, math.ceil(loop.kv_bytes[0] / (bw * t_iter)))
    res = loop.run_staggered(iters=(B + 2) * span + 2 * x, t_iter=t_iter, link_bw=bw)
    print(res, flush=True)
    assert res["verifies"] >= B and all(seen[r] >= 1 for r in range(B))
    assert res["peak_full_caches_in_hbm"] <= 2
    res = loop.run_lockstep(iters=2 * x)
    assert res["verifies"] == 2 * B
