"""ctypes binding of the C ABI in include/vc.h (argument marshalling only).

Every function takes torch tensors that already live on the GPU and passes their device
pointers; all arithmetic happens in the HIP kernels of libvc.so.  If the library is not built
the binding raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIBVC_PATH = os.path.join(PKG, "libvc.so")

VC_OK, VC_EINVAL, VC_ENOSPACE, VC_EHIP, VC_EUNSUPPORTED, VC_ENOMEM, VC_EAGAIN = 0, -1, -2, -3, -4, -5, -6
VC_EDEVICE = -7
PAGE_RESIDENT, PAGE_TRANSIENT = 0, 1
VC_VERIFY, VC_DRAFT = 0, 1
BLOCK = 16
MAX_REQS = 1024      # requests per attention launch
MAX_BATCH = 128      # requests per cache-building or commit call
MAX_ROWS = 64

# every symbol include/vc.h declares
EXPORTS = (
    "vc_attn_workspace_size", "vc_verify_attn", "vc_draft_attn", "vc_attn_mixed", "vc_attn_mixed_noalloc",
    "vc_accept",
    "vc_sample_tokens", "vc_accept_sampled",
    "vc_logits", "vc_pack_bf16", "vc_select_kept", "vc_compress", "vc_stage_kv",
    "vc_commit_rows", "vc_compress_tail", "vc_alloc_create", "vc_alloc_destroy", "vc_alloc_pages",
    "vc_alloc_release", "vc_alloc_free_count", "vc_page_row_extend", "vc_page_row_truncate",
    "vc_sched_create", "vc_sched_destroy", "vc_sched_admit", "vc_sched_advance", "vc_sched_now",
    "vc_sched_ring", "vc_sched_due",
    "vc_check_device", "vc_last_error", "vc_version",
)


class VCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vc error {code}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_rows", ctypes.c_int32)]


class Pool(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("page_table", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_sz", ctypes.c_void_p), ("v_sz", ctypes.c_void_p)]


class Commit(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("pos", ctypes.c_int32), ("count", ctypes.c_int32),
                ("page_row", ctypes.c_int32), ("kept_len", ctypes.c_int32)]


class SchedCfg(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("draft_len", ctypes.c_int32), ("t_iter", ctypes.c_double),
                ("link_bw", ctypes.c_double), ("hbm_budget", ctypes.c_double)]


class Req(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("pool", ctypes.c_int32), ("ctx_len", ctypes.c_int32),
                ("page_row", ctypes.c_int32), ("q0", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("kind", ctypes.c_int32)]


_lib = None


def lib():
    """Load libvc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBVC_PATH):
            raise ImportError(f"{LIBVC_PATH} is missing: build it with "
                              "`python -m lossless_kv_cache_vc_amd.build`")
        L = ctypes.CDLL(LIBVC_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.vc_last_error.restype = ctypes.c_char_p
        L.vc_version.restype = ctypes.c_char_p
        L.vc_attn_workspace_size.restype = sz
        L.vc_attn_workspace_size.argtypes = [P(Shape), i32, P(Req), i32]
        attn = [P(Shape), i32, P(Req), vp, vp, vp, P(Pool), vp, vp, sz, i32, vp]
        L.vc_verify_attn.argtypes = attn
        L.vc_draft_attn.argtypes = attn
        L.vc_attn_mixed.argtypes = [P(Shape), i32, P(Req), vp, vp, vp, i32, P(Pool), vp, vp, sz, i32, vp]
        L.vc_attn_mixed_noalloc.argtypes = [P(Shape), i32, P(Req), vp, vp, vp, i32, P(Pool), vp, i32, vp]
        L.vc_accept.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.vc_logits.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp]
        L.vc_sample_tokens.argtypes = [i32, i32, ctypes.c_float, vp, vp, vp, vp]
        L.vc_accept_sampled.argtypes = [i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp]
        L.vc_pack_bf16.argtypes = [P(Shape), i32, vp, i32, vp, i64, P(Pool), i32, vp]
        L.vc_select_kept.argtypes = [P(Shape), i32, vp, vp, vp, vp, i64, vp, i64, vp]
        L.vc_compress.argtypes = [P(Shape), i32, vp, P(Pool), vp, i64, P(Pool), vp]
        L.vc_stage_kv.argtypes = [vp, vp, sz, vp, vp]
        L.vc_check_device.argtypes = [vp]
        L.vc_commit_rows.argtypes = [P(Shape), i32, P(Commit), vp, vp, P(Pool), vp, i64, vp]
        L.vc_compress_tail.argtypes = [P(Shape), i32, vp, vp, P(Pool), vp, i64, P(Pool), vp]
        L.vc_alloc_create.argtypes = [ctypes.c_int32, ctypes.c_int32, P(vp)]
        L.vc_alloc_destroy.argtypes = [vp]
        L.vc_alloc_destroy.restype = None
        L.vc_alloc_pages.argtypes = [vp, i32, i32, vp]
        L.vc_alloc_release.argtypes = [vp, i32, i32, vp]
        L.vc_alloc_free_count.argtypes = [vp, i32]
        L.vc_alloc_free_count.restype = ctypes.c_int32
        L.vc_page_row_extend.argtypes = [vp, i32, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.vc_page_row_truncate.argtypes = [vp, i32, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.vc_sched_create.argtypes = [P(SchedCfg), P(vp)]
        L.vc_sched_destroy.argtypes = [vp]
        L.vc_sched_destroy.restype = None
        L.vc_sched_admit.argtypes = [vp, ctypes.c_int32, ctypes.c_double, P(ctypes.c_int64)]
        L.vc_sched_advance.argtypes = [vp]
        L.vc_sched_now.argtypes = [vp]
        L.vc_sched_now.restype = ctypes.c_int64
        L.vc_sched_ring.argtypes = [vp, ctypes.c_int32, P(ctypes.c_double), P(ctypes.c_double)]
        L.vc_sched_due.argtypes = [vp, ctypes.c_int32, vp, P(ctypes.c_int32), vp, P(ctypes.c_int32)]
        for name in EXPORTS:
            if name not in ("vc_last_error", "vc_version", "vc_attn_workspace_size", "vc_alloc_destroy",
                            "vc_alloc_free_count", "vc_sched_destroy", "vc_sched_now"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != VC_OK:
        raise VCError(rc, lib().vc_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _i32_array(vals: Sequence[int]):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


@dataclass
class PagedPool:
    """A paged KV pool: device tensors plus the page table (see vc_pool in include/vc.h)."""
    bits: int
    page_table: "object"       # int32 [rows][max_pages] (device)
    k: "object"
    v: "object"
    num_blocks: int
    k_sz: "object" = None
    v_sz: "object" = None

    def desc(self) -> Pool:
        return Pool(self.bits, int(self.page_table.shape[1]), int(self.num_blocks),
                    _ptr(self.page_table), _ptr(self.k), _ptr(self.v), _ptr(self.k_sz),
                    _ptr(self.v_sz))


def shape(L: int, Hq: int, Hkv: int, d: int, max_rows: int) -> Shape:
    return Shape(L, Hq, Hkv, d, max_rows)


def reqs_array(reqs: Sequence[Req]):
    arr = (Req * max(1, len(reqs)))()
    for i, r in enumerate(reqs):
        arr[i] = r
    return arr


def attn_workspace_size(shp: Shape, reqs: Sequence[Req], split_pages: int = 0) -> int:
    arr = reqs_array(reqs)
    return int(lib().vc_attn_workspace_size(ctypes.byref(shp), len(reqs), arr, split_pages))


def verify_attn(shp, reqs, q, blk_k, blk_v, full: PagedPool, out, workspace=None, split_pages=0,
                stream=None):
    arr = reqs_array(reqs)
    pd = full.desc()
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().vc_verify_attn(ctypes.byref(shp), len(reqs), arr, _ptr(q), _ptr(blk_k), _ptr(blk_v),
                                ctypes.byref(pd), _ptr(out), _ptr(workspace), ws, split_pages,
                                _stream(stream)))


def draft_attn(shp, reqs, q, blk_k, blk_v, comp: PagedPool, out, workspace=None, split_pages=0,
               stream=None):
    arr = reqs_array(reqs)
    pd = comp.desc()
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().vc_draft_attn(ctypes.byref(shp), len(reqs), arr, _ptr(q), _ptr(blk_k), _ptr(blk_v),
                               ctypes.byref(pd), _ptr(out), _ptr(workspace), ws, split_pages,
                               _stream(stream)))


def attn_mixed(shp, reqs, q, blk_k, blk_v, pools: Sequence[PagedPool], out, workspace=None,
               split_pages=0, stream=None):
    arr = reqs_array(reqs)
    parr = (Pool * len(pools))(*[p.desc() for p in pools])
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().vc_attn_mixed(ctypes.byref(shp), len(reqs), arr, _ptr(q), _ptr(blk_k), _ptr(blk_v),
                               len(pools), parr, _ptr(out), _ptr(workspace), ws, split_pages,
                               _stream(stream)))


SCRATCH_BYTES = 64 << 20   # the library-held workspace of attn_mixed_noalloc, per device


def attn_mixed_noalloc(shp, reqs, q, blk_k, blk_v, pools: Sequence[PagedPool], out, split_pages=0,
                       stream=None):
    arr = reqs_array(reqs)
    parr = (Pool * len(pools))(*[p.desc() for p in pools])
    _check(lib().vc_attn_mixed_noalloc(ctypes.byref(shp), len(reqs), arr, _ptr(q), _ptr(blk_k),
                                       _ptr(blk_v), len(pools), parr, _ptr(out), split_pages,
                                       _stream(stream)))


def accept(n_inst, max_x, max_xv, vocab, x, xv, draft_logits, verify_logits, draft_tok, verify_tok,
           accept_len, next_tok, stream=None):
    _check(lib().vc_accept(n_inst, max_x, max_xv, vocab, _ptr(x), _ptr(xv), _ptr(draft_logits),
                           _ptr(verify_logits), _ptr(draft_tok), _ptr(verify_tok), _ptr(accept_len),
                           _ptr(next_tok), _stream(stream)))


def sample_tokens(rows, vocab, temperature, logits, u, tokens, stream=None):
    _check(lib().vc_sample_tokens(rows, vocab, temperature, _ptr(logits), _ptr(u), _ptr(tokens),
                                  _stream(stream)))


def accept_sampled(n_inst, max_x, max_xv, vocab, temperature, x, xv, draft_logits, verify_logits,
                   draft_tok, u_accept, u_resample, accept_len, next_tok, stream=None):
    _check(lib().vc_accept_sampled(n_inst, max_x, max_xv, vocab, temperature, _ptr(x), _ptr(xv),
                                   _ptr(draft_logits), _ptr(verify_logits), _ptr(draft_tok),
                                   _ptr(u_accept), _ptr(u_resample), _ptr(accept_len), _ptr(next_tok),
                                   _stream(stream)))


def logits(rows, width, vocab, o, ld_o, w_u, z, stream=None):
    _check(lib().vc_logits(rows, width, vocab, _ptr(o), ld_o, _ptr(w_u), _ptr(z), _stream(stream)))


def pack_bf16(shp, lens, layer, src, src_rows, pool: PagedPool, which, stream=None):
    pd = pool.desc()
    _check(lib().vc_pack_bf16(ctypes.byref(shp), len(lens), _i32_array(lens), layer, _ptr(src),
                              src_rows, ctypes.byref(pd), which, _stream(stream)))


def select_kept(shp, lens, recent, top, scores, score_stride, kept, kept_stride, stream=None):
    _check(lib().vc_select_kept(ctypes.byref(shp), len(lens), _i32_array(lens), _i32_array(recent),
                                _i32_array(top), _ptr(scores), score_stride, _ptr(kept), kept_stride,
                                _stream(stream)))


def compress(shp, comp_lens, src: PagedPool, kept, kept_stride, dst: PagedPool, stream=None):
    sd, dd = src.desc(), dst.desc()
    _check(lib().vc_compress(ctypes.byref(shp), len(comp_lens), _i32_array(comp_lens), ctypes.byref(sd),
                             _ptr(kept), kept_stride, ctypes.byref(dd), _stream(stream)))


def stage_kv(dst, src_pinned, nbytes, side_stream, event=None):
    """event: a torch.cuda.Event that has been recorded once (torch creates the HIP event on its
    first record; before that it has no handle to pass)."""
    ev = None if event is None else event.cuda_event
    if event is not None and not ev:
        raise ValueError("stage_kv: the event has no HIP handle yet; record it once first")
    _check(lib().vc_stage_kv(_ptr(dst), _ptr(src_pinned), nbytes, _stream(side_stream), ev))


def check_device(stream=None):
    """Synchronise `stream` and raise VCError(VC_EDEVICE) if a kernel met a corrupt page-table
    entry since the last check (the device error word is then cleared)."""
    _check(lib().vc_check_device(_stream(stream)))


def version() -> str:
    return lib().vc_version().decode()


def commit_rows(shp, commits, blk_k, blk_v, pool: "PagedPool", kept=None, kept_stride=0, stream=None):
    """commits: (slot, pos, count, page_row, kept_len) per request."""
    arr = (Commit * max(1, len(commits)))(*[Commit(*c) for c in commits])
    pd = pool.desc()
    _check(lib().vc_commit_rows(ctypes.byref(shp), len(commits), arr, _ptr(blk_k), _ptr(blk_v),
                                ctypes.byref(pd), _ptr(kept), kept_stride, _stream(stream)))


def compress_tail(shp, from_lens, comp_lens, src: "PagedPool", kept, kept_stride, dst: "PagedPool",
                  stream=None):
    sd, dd = src.desc(), dst.desc()
    _check(lib().vc_compress_tail(ctypes.byref(shp), len(comp_lens), _i32_array(from_lens),
                                  _i32_array(comp_lens), ctypes.byref(sd), _ptr(kept), kept_stride,
                                  ctypes.byref(dd), _stream(stream)))


class PageAllocator:
    """Host page allocator of the library (resident ids [0, num_resident), transient ids above)."""

    def __init__(self, num_blocks: int, num_resident: int):
        h = ctypes.c_void_p()
        _check(lib().vc_alloc_create(num_blocks, num_resident, ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().vc_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def alloc(self, kind: int, n: int):
        ids = (ctypes.c_int32 * max(1, n))()
        _check(lib().vc_alloc_pages(self._h, kind, n, ids))
        return list(ids[:n])

    def release(self, kind: int, ids):
        arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
        _check(lib().vc_alloc_release(self._h, kind, len(ids), arr))

    def free_count(self, kind: int) -> int:
        return int(lib().vc_alloc_free_count(self._h, kind))

    def extend_row(self, kind: int, row, old_len: int, new_len: int):
        """row: a C-contiguous numpy int32 array (one request's page-table row), updated in place."""
        _check(lib().vc_page_row_extend(self._h, kind, row.ctypes.data, len(row), old_len, new_len))

    def truncate_row(self, kind: int, row, old_len: int, new_len: int):
        _check(lib().vc_page_row_truncate(self._h, kind, row.ctypes.data, len(row), old_len, new_len))


class Scheduler:
    """The library's Admit scheduler (link and HBM rings over a lookahead window)."""

    def __init__(self, window: int, draft_len: int, t_iter: float, link_bw: float, hbm_budget: float):
        self.cfg = SchedCfg(window, draft_len, t_iter, link_bw, hbm_budget)
        h = ctypes.c_void_p()
        _check(lib().vc_sched_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().vc_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def admit(self, req: int, kv_full_bytes: float) -> Optional[int]:
        """The reserved verify iteration, or None when nothing fits now."""
        out = ctypes.c_int64()
        rc = lib().vc_sched_admit(self._h, req, kv_full_bytes, ctypes.byref(out))
        if rc == VC_EAGAIN:
            return None
        _check(rc)
        return int(out.value)

    def advance(self):
        _check(lib().vc_sched_advance(self._h))

    @property
    def now(self) -> int:
        return int(lib().vc_sched_now(self._h))

    def ring(self, i: int):
        a, b = ctypes.c_double(), ctypes.c_double()
        _check(lib().vc_sched_ring(self._h, i, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def due(self, cap: int = 1024):
        r = (ctypes.c_int32 * cap)()
        v = (ctypes.c_int32 * cap)()
        nr, nv = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().vc_sched_due(self._h, cap, r, ctypes.byref(nr), v, ctypes.byref(nv)))
        return list(r[:nr.value]), list(v[:nv.value])
