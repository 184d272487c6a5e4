"""Byte accounting of the method (pure arithmetic).

Sources
-------
* VeriCache review, §Prerequisites "Transformer attention and the KV cache": KV size
  = 2 * n * L * h * d_h * b bytes (about 13 GB for Llama-3.1-8B at 100K context).
* Same page, §Theoretical Analysis, Eq. (3) and "Step-by-step derivation of T_iter": per
  iteration HBM bytes = M + B * KV_full * (c + 1/x); interconnect bytes = (B / x) * KV_full.
* Same page, §KV Swap Scheduling "Concrete numbers from the paper": one 4 GB full-KV transfer
  over a 64 GB/s link takes 62.5 ms.
* Same page, §Theoretical Analysis, Eq. (3) itself: T_iter is the larger of the HBM time
  T_gpu = HBM bytes / BW_hbm and the link time T_xfer = link bytes / BW_inter; and the
  acceptance model: eta = 1 + gamma * x / (x + 1) tokens per request per iteration, throughput
  eta / T_iter per request (times B for the batch, as in the worked examples).
* The crossover compression c* is the c at which the two terms of Eq. (3) are equal.  Solving
  Eq. (3) gives (rho - 1) / x - M / (B * KV_full), with rho = BW_hbm / BW_inter; the
  expression printed on the page does not satisfy that equality (a garble), so the oracle
  solves Eq. (3) instead.
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


def iteration_time(M: float, B: int, kv_full: float, c: float, x: int, bw_hbm: float,
                   bw_inter: float):
    """Eq. (3): (T_gpu, T_xfer, T_iter) of one iteration of the staggered schedule."""
    t_gpu = transfer_seconds(iteration_hbm_bytes(M, B, kv_full, c, x), bw_hbm)
    t_xfer = transfer_seconds(iteration_link_bytes(B, kv_full, x), bw_inter)
    return t_gpu, t_xfer, max(t_gpu, t_xfer)


def crossover_compression(M: float, B: int, kv_full: float, x: int, bw_hbm: float,
                          bw_inter: float) -> float:
    """The c that makes the two terms of Eq. (3) equal:
    (M + B*KV*(c + 1/x)) / BW_hbm = B*KV / (x * BW_inter), solved for c."""
    return (bw_hbm * B * kv_full / (x * bw_inter) - M) / (B * kv_full) - 1.0 / x


def effective_tokens(gamma: float, x: int) -> float:
    """Acceptance model: eta = 1 + gamma * x / (x + 1)."""
    return 1.0 + gamma * x / (x + 1)


def batch_tokens_per_second(B: int, gamma: float, x: int, t_iter: float) -> float:
    """B requests, each eta tokens per iteration of T_iter seconds."""
    return B * effective_tokens(gamma, x) / t_iter
