"""Byte accounting of the method (pure arithmetic).

Sources
-------
* VeriCache review, §Prerequisites "Transformer attention and the KV cache": KV size
  = 2 * n * L * h * d_h * b bytes (about 13 GB for Llama-3.1-8B at 100K context).
* Same page, §Theoretical Analysis, Eq. (3) and "Step-by-step derivation of T_iter": per
  iteration HBM bytes = M + B * KV_full * (c + 1/x); interconnect bytes = (B / x) * KV_full.
* Same page, §KV Swap Scheduling "Concrete numbers from the paper": one 4 GB full-KV transfer
  over a 64 GB/s link takes 62.5 ms.
"""
from __future__ import annotations


def kv_bytes(n: int, L: int, h: int, d: int, b: int) -> int:
    """Bytes of K and V for n tokens, L layers, h KV heads of size d, b bytes per element."""
    return 2 * n * L * h * d * b


def iteration_hbm_bytes(M: float, B: int, kv_full: float, c: float, x: int) -> float:
    """Eq. (3) numerator: weights once, B drafters' compressed caches, one amortised verify."""
    return M + B * kv_full * (c + 1.0 / x)


def iteration_link_bytes(B: int, kv_full: float, x: int) -> float:
    """Eq. (3) transfer term numerator: one full KV per request every x iterations."""
    return B * kv_full / x


def transfer_seconds(nbytes: float, bw_bytes_per_s: float) -> float:
    return nbytes / bw_bytes_per_s
