"""Iteration-time and throughput model of staggered draft/verify serving, fed by MI355X numbers.

Follows "VeriCache" (throughput model for long-context decoding, Eq. 3, and the acceptance
model that follows it).  Per iteration of the staggered schedule, B requests draft one token
each over their compressed caches (c of the full size), and about B/x of them verify x tokens
over the full cache.  So HBM carries the weights M once plus B*KV_full*(c + 1/x) bytes of
cache, and the host link must deliver one full cache per request every x iterations:

    T_gpu  = (M + B*KV_full*(c + 1/x)) / BW_hbm
    T_xfer = B*KV_full / (x*BW_inter)
    T_iter = max(T_gpu, T_xfer)           (staggering overlaps the two)

    eta    = 1 + gamma*x/(x + 1)           effective tokens per request per iteration
    tokens/s = B*eta / T_iter

Crossover.  Setting T_gpu = T_xfer in Eq. 3 gives c* = (rho - 1)/x - M/(B*KV_full), with
rho = BW_hbm/BW_inter: below c* the host link binds, above it HBM does.  The pages print a
different expression with the opposite reading; the function here follows Eq. 3 itself.

Units: bytes, bytes per second, seconds.  This is host-side arithmetic only.

    python -m lossless_kv_cache_vc_amd.throughput --bench BENCH.json [--stage-gbps 57]
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import asdict, dataclass
from typing import Optional

GB = 1e9


@dataclass
class IterTime:
    hbm_bytes: float   # M + B*KV_full*(c + 1/x)
    xfer_bytes: float  # B*KV_full/x
    t_gpu: float
    t_xfer: float
    t_iter: float
    bound: str         # "hbm" or "interconnect"


def t_iter(M: float, B: int, kv_full: float, c: float, x: int, bw_hbm: float,
           bw_inter: float) -> IterTime:
    """Eq. 3: iteration time of the staggered schedule (the larger of HBM and link time)."""
    if x <= 0 or B <= 0 or bw_hbm <= 0 or bw_inter <= 0:
        raise ValueError("x, B and both bandwidths must be positive")
    hbm = M + B * kv_full * (c + 1.0 / x)
    xfer = B * kv_full / x
    tg, tx = hbm / bw_hbm, xfer / bw_inter
    return IterTime(hbm, xfer, tg, tx, max(tg, tx), "hbm" if tg >= tx else "interconnect")


def c_star(rho: float, x: int, m_over_bkv: float) -> float:
    """Compression ratio at which the two terms of Eq. 3 are equal (re-derived from Eq. 3)."""
    return (rho - 1.0) / x - m_over_bkv


def eta(gamma: float, x: int) -> float:
    """Effective tokens per request per iteration: 1 + gamma*x/(x + 1)."""
    return 1.0 + gamma * x / (x + 1.0)


def tokens_per_s(B: int, eta_value: float, t_iter_s: float) -> float:
    return B * eta_value / t_iter_s


def from_bench(bench: dict, stage_gbps: float, M: float = 0.0, gamma: Optional[float] = None,
               peak_gbps: float = 8000.0) -> dict:
    """Eq. 3 at a measured workload.

    The bench line gives B, x, the per-step draft and verify bytes, and the measured kernel
    times.  KV_full is the verify bytes per request and c the draft/verify byte ratio.  T_gpu
    is predicted at peak HBM and at the measured draft and verify rates; the measured iteration
    (one draft launch plus 1/x of a verify) is reported beside both.  T_xfer uses the measured
    host-to-device staging rate."""
    cfg, by, br = bench["config"], bench["bytes"], bench["breakdown_ms"]
    B, x = int(cfg["batch"]), int(cfg["x"])
    kv_full = by["verify"] / B
    c = by["draft_per_step_avg"] / by["verify"]
    bw_inter = stage_gbps * GB
    peak = t_iter(M, B, kv_full, c, x, peak_gbps * GB, bw_inter)
    draft_bw = by["draft_per_step_avg"] / (br["draft_per_launch"] * 1e-3)
    verify_bw = by["verify"] / (br["verify"] * 1e-3)
    # the measured iteration: one draft launch and 1/x of a verify launch
    t_meas = (br["draft_per_launch"] + br["verify"] / x) * 1e-3
    # Eq. 3's HBM term at the measured kernel rates (each byte class at its own rate)
    t_gpu_meas = M / (peak_gbps * GB) + B * kv_full * c / draft_bw + B * kv_full / x / verify_bw
    out = {
        "workload": cfg.get("workload"), "B": B, "x": x, "kv_full_GB": kv_full / GB, "c": c,
        "M_GB": M / GB, "rho_peak": peak_gbps * GB / bw_inter,
        "rho_measured": (B * kv_full * (c + 1.0 / x)) / t_meas / bw_inter,
        "c_star_peak": c_star(peak_gbps * GB / bw_inter, x, M / (B * kv_full)),
        "eq3_at_peak_hbm": asdict(peak),
        "t_gpu_at_measured_rates_s": t_gpu_meas,
        "t_iter_measured_gpu_s": t_meas,
        "t_xfer_s": peak.t_xfer,
        "bound_measured": "hbm" if t_meas >= peak.t_xfer else "interconnect",
    }
    if gamma is not None:
        e = eta(gamma, x)
        out["eta"] = e
        out["tokens_per_s_eq3_peak"] = tokens_per_s(B, e, peak.t_iter)
        out["tokens_per_s_measured_gpu"] = tokens_per_s(B, e, max(t_meas, peak.t_xfer))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--bench", required=True, help="one JSON line written by bench.py")
    ap.add_argument("--stage-gbps", type=float, default=57.0,
                    help="measured pinned host -> HBM staging rate (GB/s)")
    ap.add_argument("--weights-gb", type=float, default=0.0, help="model weight bytes M (GB)")
    ap.add_argument("--gamma", type=float, default=None, help="acceptance rate for eta")
    args = ap.parse_args(argv)
    line = open(args.bench).read().strip().splitlines()[-1]
    print(json.dumps(from_bench(json.loads(line), args.stage_gbps, args.weights_gb * GB, args.gamma), indent=1))


if __name__ == "__main__":
    sys.exit(main())
