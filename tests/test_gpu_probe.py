"""The streaming-read probe reads the whole buffer (checksum = XOR of its words) and reports a
rate (run on an MI355X: -m gpu)."""
import numpy as np
import pytest
import torch

from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def test_read_reads_the_whole_buffer():
    require_gpu()
    from lossless_kv_cache_vc_amd import stream_probe as sp
    host = np.random.default_rng(8).integers(0, 256, size=(1 << 22) + 16 * 37, dtype=np.uint8)  # ragged tail
    buf = torch.from_numpy(host).cuda()
    want = int(np.bitwise_xor.reduce(host.view(np.uint32)))
    for groups in (1, 64, 2048):
        cs = torch.zeros(groups, dtype=torch.int32, device="cuda")
        print(f"streaming read groups={groups}", flush=True)
        sp.read(buf, cs, groups=groups)
        torch.cuda.synchronize()
        assert sp.xor_all(cs, groups) == want


def test_probe_measures_a_rate():
    require_gpu()
    from lossless_kv_cache_vc_amd import stream_probe as sp
    r = sp.measure(gib=0.5, reps=2)
    assert 100 < r["read_gbps"] < 10000, r
