"""GPU side of the seeded generator: fills dense torch tensors on the device with the same bits
that :mod:`vcsynth.rng` / :mod:`vcsynth.tensors` produce on the CPU."""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Sequence

import numpy as np

from .normal_table import normal_table

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvcsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build with `python -m lossless_kv_cache_vc_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
        P64 = ctypes.POINTER(ctypes.c_int64)
        L.vcs_fill_normal_bf16.argtypes = [vp, i32, P64, P64, i64, u64, u32, vp, vp, i32, vp]
        L.vcs_fill_normal_bf16.restype = i32
        L.vcs_fill_u32.argtypes = [vp, i32, P64, P64, i64, u64, u32, vp]
        L.vcs_fill_u32.restype = i32
        _lib = L
    return _lib


@functools.lru_cache(maxsize=None)
def _table_on(device_index: int, sigma: float):
    import torch
    t = normal_table(sigma)
    thr = torch.from_numpy(t.thresholds.view(np.int32).copy()).to(f"cuda:{device_index}")
    val = torch.from_numpy(t.values_bits.view(np.int16).copy()).to(f"cuda:{device_index}")
    return thr, val, len(t.thresholds)


def _arr(vals: Sequence[int]):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_normal_bf16(dst, lstrides: Sequence[int], lbase: int, seed: int, stream_id: int,
                     sigma: float = 1.0):
    """Fill the contiguous tensor ``dst`` (bfloat16 or int16 storage) with N(0, sigma^2) bf16 draws;
    element with coordinates c gets logical index lbase + sum c_k * lstrides[k]."""
    assert dst.is_contiguous() and dst.element_size() == 2
    shape = list(dst.shape)
    assert len(shape) == len(lstrides)
    thr, val, ntab = _table_on(dst.device.index or 0, float(sigma))
    rc = lib().vcs_fill_normal_bf16(dst.data_ptr(), len(shape), _arr(shape), _arr(lstrides), int(lbase),
                                    int(seed), int(stream_id), thr.data_ptr(), val.data_ptr(), ntab,
                                    _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"vcs_fill_normal_bf16 failed ({rc})")


def fill_u32(dst, lstrides: Sequence[int], lbase: int, seed: int, stream_id: int):
    """Fill the contiguous 32-bit tensor ``dst`` with raw upper-32-bit draws."""
    assert dst.is_contiguous() and dst.element_size() == 4
    shape = list(dst.shape)
    rc = lib().vcs_fill_u32(dst.data_ptr(), len(shape), _arr(shape), _arr(lstrides), int(lbase),
                            int(seed), int(stream_id), _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"vcs_fill_u32 failed ({rc})")
