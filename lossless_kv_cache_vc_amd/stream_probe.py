"""Streaming-read peak of this GPU (a measurement, not part of the method): coalesced
nontemporal 16-byte vector loads over a contiguous buffer (``libvcprobe.so``).  The benchmark
reports its kernels' rates against this peak next to the nominal 8 TB/s.

    python -m lossless_kv_cache_vc_amd.stream_probe --gib 8 --reps 5
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIBPROBE_PATH = os.path.join(PKG, "libvcprobe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPROBE_PATH):
            raise ImportError(f"{LIBPROBE_PATH} is missing: build it with python -m lossless_kv_cache_vc_amd.build")
        L = ctypes.CDLL(LIBPROBE_PATH)
        L.vcprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
        L.vcprobe_read.restype = ctypes.c_int
        _lib = L
    return _lib


def read(buf, checksum, groups: int = 2048, stream=None) -> None:
    """One streaming read of the whole of ``buf`` (device tensor, a multiple of 16 bytes);
    ``checksum`` (at least ``groups`` int32) receives each work-group's XOR of the words it read
    (see ``xor_all``)."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if checksum.numel() < groups:
        raise ValueError("checksum needs one word per work-group")
    s = torch.cuda.current_stream() if stream is None else stream
    rc = lib().vcprobe_read(buf.data_ptr(), nbytes, groups, checksum.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"vcprobe_read failed ({rc})")


def xor_all(checksum, words: int) -> int:
    """XOR of the first ``words`` checksum words (host integer)."""
    w = checksum[:words].cpu().numpy().view(np.uint32)
    return int(np.bitwise_xor.reduce(w)) if w.size else 0


def measure(gib: float = 4.0, reps: int = 3, groups: int = 2048, device: str = "cuda") -> dict:
    """GB/s of a ``gib`` GiB streaming read (mean of ``reps`` launches after one warm-up)."""
    import torch
    nbytes = int(gib * (1 << 30)) // 16 * 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(0x5A)
    checksum = torch.zeros(groups, dtype=torch.int32, device=device)
    read(buf, checksum, groups)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        read(buf, checksum, groups)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del buf
    torch.cuda.empty_cache()
    return {"kind": "contiguous nontemporal 16-byte vector loads", "buffer_bytes": nbytes, "reps": reps,
            "read_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description="streaming-read peak of this GPU")
    ap.add_argument("--gib", type=float, default=8.0)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args(argv)
    print(json.dumps(measure(args.gib, args.reps)), flush=True)


if __name__ == "__main__":
    main()
