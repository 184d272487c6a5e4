import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# every tensor the kernels write gets guard regions in the GPU tests (lossless_kv_cache_vc_amd
# harness), checked after each test
os.environ.setdefault("VC_CANARY", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _guard_regions_intact(request):
    """After each GPU test, every workload's guard regions must be untouched (no write past the
    ends of a pool, output, workspace, kept list or logits tensor)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    mod = sys.modules.get("lossless_kv_cache_vc_amd.harness")
    if mod is not None:
        mod.check_all_canaries()
