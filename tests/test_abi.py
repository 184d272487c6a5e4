"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from lossless_kv_cache_vc_amd import vc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "vc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vc_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(vc.EXPORTS)


def test_library_exports_every_symbol():
    lib = vc.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert vc.version().startswith("vc ")


def _shape(**kw):
    s = dict(L=2, Hq=8, Hkv=2, d=128, max_rows=32)
    s.update(kw)
    return vc.shape(s["L"], s["Hq"], s["Hkv"], s["d"], s["max_rows"])


class _FakeTensor:
    """Something with a data_ptr(): host validation never dereferences device pointers."""
    def __init__(self, addr, shape=(1, 4)):
        self.addr, self.shape = addr, shape

    def data_ptr(self):
        return self.addr


def _pool(bits=16):
    t = _FakeTensor(0x1000, (4, 8))
    return vc.PagedPool(bits, t, t, t, 16, t if bits != 16 else None, t if bits != 16 else None)


def _expect(code, fn):
    with pytest.raises(vc.VCError) as e:
        fn()
    assert e.value.code == code, str(e.value)


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device pointers; host-only check")
def test_host_validation_rejects_bad_arguments():
    t = _FakeTensor(0x1000)
    ok_req = vc.Req(0, 0, 100, 0, 0, 8, vc.VC_VERIFY)
    call = lambda shp, reqs, pool=_pool(), ws=None: vc.verify_attn(shp, reqs, t, t, t, pool, t, ws, 0, 0)
    _expect(vc.VC_EUNSUPPORTED, lambda: call(_shape(d=96), [ok_req]))
    _expect(vc.VC_EINVAL, lambda: call(_shape(Hq=6, Hkv=4), [ok_req]))
    _expect(vc.VC_EINVAL, lambda: call(_shape(max_rows=24), [ok_req]))
    _expect(vc.VC_EINVAL, lambda: call(_shape(), [vc.Req(0, 0, 100, 0, 30, 8, vc.VC_VERIFY)]))  # q0+rows > max
    _expect(vc.VC_EINVAL, lambda: call(_shape(), [vc.Req(0, 0, -1, 0, 0, 8, vc.VC_VERIFY)]))
    _expect(vc.VC_EINVAL, lambda: call(_shape(), [vc.Req(0, 0, 16 * 9, 0, 0, 8, vc.VC_VERIFY)]))  # > max_pages
    _expect(vc.VC_EINVAL, lambda: call(_shape(), [ok_req], pool=_pool(bits=3)))
    _expect(vc.VC_EINVAL, lambda: call(_shape(), [ok_req], pool=_pool(bits=2)))  # verify needs bf16
    _expect(vc.VC_EINVAL, lambda: vc.draft_attn(_shape(Hq=32, Hkv=2), [vc.Req(0, 0, 10, 0, 0, 2, 1)],
                                                 t, t, t, _pool(), t, None, 0, 0))  # rows*G > 16
    _expect(vc.VC_EINVAL, lambda: vc.verify_attn(_shape(), [ok_req], t, t, t, _pool(), t, None, 6, 0))
    # a KIVI pool whose one layer of 512-byte page arrays reaches 2^32 bytes (2^22 blocks x 2 kv
    # heads x 512 B) is refused; L x blocks x kv heads (2^24) is within its own limit
    big = _pool(bits=2)
    big.num_blocks = 1 << 22
    draft_req = vc.Req(0, 0, 100, 0, 0, 1, vc.VC_DRAFT)
    _expect(vc.VC_EUNSUPPORTED, lambda: vc.draft_attn(_shape(), [draft_req], t, t, t, big, t, None, 0, 0))
    # splitting needs a workspace
    _expect(vc.VC_ENOSPACE, lambda: vc.verify_attn(_shape(), [vc.Req(0, 0, 120, 0, 0, 8, 0)], t, t, t,
                                                   _pool(), t, None, 4, 0))
    _expect(vc.VC_EINVAL, lambda: vc.accept(1, 65, 65, 10, t, t, t, t, t, t, t, t, 0))
    _expect(vc.VC_EINVAL, lambda: vc.logits(4, 8, 8, t, 4, t, t, 0))


def test_empty_launches_do_nothing():
    """Launches with nothing to compute return VC_OK without touching the device (this runs
    without a GPU): no requests, no rows of logits, no accept instances."""
    t = _FakeTensor(0x1000)
    vc.verify_attn(_shape(), [], t, t, t, _pool(), t, None, 0, 0)
    vc.draft_attn(_shape(), [], t, t, t, _pool(), t, None, 0, 0)
    vc.attn_mixed(_shape(), [], t, t, t, [_pool(), _pool()], t, None, 0, 0)
    vc.logits(0, 8, 8, t, 8, t, t, 0)
    vc.accept(0, 4, 4, 16, t, t, t, t, t, t, t, t, 0)
    assert vc.attn_workspace_size(_shape(), []) == 0
    # rows must be at least 1 and fit the drafted-block capacity even when nothing else is wrong
    _expect(vc.VC_EINVAL, lambda: vc.verify_attn(_shape(), [vc.Req(0, 0, 100, 0, 0, 0, vc.VC_VERIFY)],
                                                 t, t, t, _pool(), t, None, 0, 0))


def test_workspace_size_accounts_for_splits():
    shp = _shape()
    r = vc.Req(0, 0, 16 * 100, 0, 0, 8, vc.VC_VERIFY)
    assert vc.attn_workspace_size(shp, [r], 400) == 0            # one split
    # 100 pages in chunks of 40 -> 3 splits of 8 rows * 4 heads, d + 4 floats each
    assert vc.attn_workspace_size(shp, [r], 40) == 2 * 2 * 3 * 8 * 4 * 132 * 4


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device pointers; host-only check")
def test_sampling_entry_points_validate_on_host():
    t = _FakeTensor(0x1000)
    z = _FakeTensor(0)
    _expect(vc.VC_EINVAL, lambda: vc.sample_tokens(-1, 16, 0.7, t, t, t, 0))
    _expect(vc.VC_EINVAL, lambda: vc.sample_tokens(4, 0, 0.7, t, t, t, 0))
    _expect(vc.VC_EINVAL, lambda: vc.sample_tokens(4, 16, 0.0, t, t, t, 0))
    _expect(vc.VC_EINVAL, lambda: vc.sample_tokens(4, 16, float("inf"), t, t, t, 0))
    _expect(vc.VC_EINVAL, lambda: vc.sample_tokens(4, 16, 0.7, t, z, t, 0))
    vc.sample_tokens(0, 16, 0.7, t, t, t, 0)  # nothing to do: no launch, no error
    acc = lambda n=2, mx=4, mxv=5, V=16, T=0.7, u=t: vc.accept_sampled(n, mx, mxv, V, T, t, t, t, t, t, t, u, t, t, 0)
    _expect(vc.VC_EINVAL, lambda: acc(n=-1))
    _expect(vc.VC_EINVAL, lambda: acc(mx=0))
    _expect(vc.VC_EINVAL, lambda: acc(mx=65))
    _expect(vc.VC_EINVAL, lambda: acc(mxv=66))
    _expect(vc.VC_EINVAL, lambda: acc(V=0))
    _expect(vc.VC_EINVAL, lambda: acc(T=-1.0))
    _expect(vc.VC_EINVAL, lambda: acc(u=z))
    acc(n=0)


def test_stream_probe_library_loads_and_rejects_bad_arguments():
    """The streaming-read probe (a measurement library beside libvc) loads without a GPU and
    refuses bad arguments before launching anything."""
    from lossless_kv_cache_vc_amd import stream_probe as sp
    L = sp.lib()
    assert L.vcprobe_read(None, 16, 1, 0x3000, None) == -1
    assert L.vcprobe_read(0x1000, 0, 1, 0x3000, None) == -1                      # nothing to read
    assert L.vcprobe_read(0x1000, 24, 1, 0x3000, None) == -1                     # not 16-byte pieces
    assert L.vcprobe_read(0x1000, 16, 0, 0x3000, None) == -1                     # no groups
    assert L.vcprobe_read(0x1000, 16, 1, None, None) == -1


def test_status_codes_and_limits_agree_with_the_header():
    src = open(os.path.join(ROOT, "include", "vc.h")).read()
    codes = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"\b(VC_E[A-Z]+|VC_OK)\s*=\s*(-?\d+)", src))
    for name, val in codes.items():
        assert getattr(vc, name) == val, name
    assert codes["VC_EDEVICE"] == -7
    limits = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"#define (VC_MAX_[A-Z]+) (\d+)", src))
    assert limits == {"VC_MAX_REQS": vc.MAX_REQS, "VC_MAX_BATCH": vc.MAX_BATCH, "VC_MAX_ROWS": vc.MAX_ROWS}


def test_workspace_holds_the_request_table_of_large_launches():
    """More than 64 requests: the launch's request table (56 bytes per request, rounded up to
    256) heads the workspace, before any split partials; 64 or fewer ride in the kernel
    arguments."""
    shp = _shape()
    r = vc.Req(0, 0, 16 * 10, 0, 0, 8, vc.VC_VERIFY)
    assert vc.attn_workspace_size(shp, [r] * 64, 400) == 0
    assert vc.attn_workspace_size(shp, [r] * 65, 400) == (65 * 56 + 255) // 256 * 256
    assert vc.attn_workspace_size(shp, [r] * 1024, 400) == 1024 * 56
    assert vc.attn_workspace_size(shp, [r] * 1025, 400) == 0          # rejected
    split = vc.attn_workspace_size(shp, [r], 4)                         # 3 splits of one request
    assert vc.attn_workspace_size(shp, [r] * 100, 4) == (100 * 56 + 255) // 256 * 256 + 100 * split


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device pointers; host-only check")
def test_large_launches_validate_on_host():
    t = _FakeTensor(0x1000)
    r = vc.Req(0, 0, 100, 0, 0, 8, vc.VC_VERIFY)
    _expect(vc.VC_EINVAL, lambda: vc.verify_attn(_shape(), [r] * 1025, t, t, t, _pool(), t, None, 0, 0))
    # 65 requests need the workspace for their table
    _expect(vc.VC_ENOSPACE, lambda: vc.verify_attn(_shape(), [r] * 65, t, t, t, _pool(), t, None, 0, 0))
    ws = _FakeTensor(0x2000, (16,))
    ws.numel, ws.element_size = (lambda: 16), (lambda: 4)   # 64 bytes: too small
    _expect(vc.VC_ENOSPACE, lambda: vc.verify_attn(_shape(), [r] * 65, t, t, t, _pool(), t, ws, 0, 0))
    # build and commit calls take at most 128 requests
    _expect(vc.VC_EINVAL, lambda: vc.compress(_shape(), [16] * 129, _pool(), None, 0, _pool(), 0))
    _expect(vc.VC_EINVAL, lambda: vc.select_kept(_shape(), [16] * 129, [0] * 129, [4] * 129, t, 16, t, 16, 0))
    _expect(vc.VC_EINVAL, lambda: vc.commit_rows(_shape(), [(0, 0, 1, 0, 0)] * 129, t, t, _pool(), None, 0, 0))


def test_stage_kv_checks_its_arguments_on_the_host():
    """bytes == 0 enqueues no copy (and, without an event, touches no device); NULL pointers with
    bytes > 0 are rejected before any HIP call."""
    lib = vc.lib()
    assert lib.vc_stage_kv(None, None, 0, None, None) == vc.VC_OK
    assert lib.vc_stage_kv(None, 0x1000, 64, None, None) == vc.VC_EINVAL
    assert lib.vc_stage_kv(0x1000, None, 64, None, None) == vc.VC_EINVAL


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device pointers; host-only check")
def test_noalloc_launch_refuses_on_the_host():
    """vc_attn_mixed_noalloc sizes its launch before touching a device: beyond the library's
    scratch array (VC_SCRATCH_BYTES) it returns VC_ENOSPACE; with nothing to do it returns OK."""
    t = _FakeTensor(0x1000)
    shp = _shape(max_rows=16)
    r = vc.Req(0, 0, 16 * 8, 0, 0, 8, vc.VC_VERIFY)
    many = [r] * 1024                      # 2 splits x 2 kv heads x 32 rows x 132 floats each
    assert vc.attn_workspace_size(shp, many, 4) > vc.SCRATCH_BYTES
    _expect(vc.VC_ENOSPACE, lambda: vc.attn_mixed_noalloc(shp, many, t, t, t, [_pool()], t, 4, 0))
    vc.attn_mixed_noalloc(shp, [], t, t, t, [_pool()], t, 0, 0)
    _expect(vc.VC_EINVAL, lambda: vc.attn_mixed_noalloc(shp, [r] * 1025, t, t, t, [_pool()], t, 0, 0))
