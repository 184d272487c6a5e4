"""Pinned host buffers of an exact size (hipHostMalloc), for keeping a full KV cache in host memory
between its reloads.

PyTorch's pinned allocator rounds every request up to a power of two, which would nearly double
the host memory of a 34 GB cache half; these buffers take exactly what is asked.  A buffer is
viewed as a CPU tensor without a copy; it stays valid while the PinnedBuffer lives.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

_hip = None


def _lib():
    global _hip
    if _hip is None:
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        lib.hipHostMalloc.restype = ctypes.c_int
        lib.hipHostFree.argtypes = [ctypes.c_void_p]
        lib.hipHostFree.restype = ctypes.c_int
        _hip = lib
    return _hip


class PinnedBuffer:
    """nbytes of page-locked host memory (default hipHostMalloc flags: portable, coherent)."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        p = ctypes.c_void_p()
        rc = _lib().hipHostMalloc(ctypes.byref(p), self.nbytes, 0)
        if rc != 0 or not p.value:
            raise MemoryError(f"hipHostMalloc of {self.nbytes} bytes failed (error {rc})")
        self.ptr = p.value

    def tensor(self, dtype: torch.dtype, shape) -> torch.Tensor:
        """A CPU tensor over the buffer (no copy)."""
        arr = np.ctypeslib.as_array(ctypes.cast(self.ptr, ctypes.POINTER(ctypes.c_uint8)), shape=(self.nbytes,))
        t = torch.from_numpy(arr).view(dtype)
        return t.view(shape)

    def free(self):
        if self.ptr:
            _lib().hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass
