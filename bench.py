#!/usr/bin/env python3
"""Benchmark of the draft/verify attention hot path on one MI355X.

One step is one draft-verify round over the whole batch of the Llama-3.1-8B 32K workload
(8 requests, 32 layer slices, 32 query / 8 KV heads, d = 128, n = 32768, x = 32, 4x token
drop): x single-query draft launches over the compressed cache, one verify launch over the full
cache, the LM-head stand-in for both, and the greedy accept.  Inputs are resident in HBM before
the timed region.  The metric is the attention's achieved HBM bandwidth: algorithmic bytes of
the draft and verify launches divided by their measured time.

    python bench.py [--steps K] [--warmup W] [--config C2] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
METRIC = "verify+draft attention achieved HBM TB/s (% of peak), Llama-3.1-8B shape 32K"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def measured_traffic(config: str, kind: str):
    """HBM bytes per launch of one attention kernel of one workload from the committed rocprofv3
    counter runs (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or None when
    absent or taken on other kernel code."""
    from lossless_kv_cache_vc_amd.profiling import attn_source_hash
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != attn_source_hash():
        return None
    k = rec.get("configs", {}).get(config, {}).get("kernels", {}).get(kind)
    return None if not k else k.get("bytes_per_launch")


def host_info():
    """The host the oracle ran on: CPU model, logical CPUs usable by this process, RAM."""
    model, ram_gb = None, None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kb = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal")), None)
        ram_gb = None if kb is None else round(kb / 2**20, 1)
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": usable, "ram_gib": ram_gb}


def cpu_baseline(cfg, budget_s: float):
    """The oracle, untuned, on a bounded sample of the same round, scaled to the whole round:
    (request, layer, kv head) units of the verify pass plus all x draft steps are timed until
    about `budget_s` seconds of oracle work have run, plus one instance's logits and accept."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    from oracle import accept as oacc
    from oracle import attention as oatt
    from oracle import workload as ow

    G, x = cfg.G, cfg.reqs[0].x
    t_units, units = 0.0, 0
    while t_units < budget_s and units < cfg.B * cfg.L * cfg.Hkv:
        r, l, g = units % cfg.B, (7 * units) % cfg.L, (3 * units) % cfg.Hkv
        q = ow.queries(cfg, r, l, x)[:, g * G:(g + 1) * G]
        kc, vc = ow.context(cfg, r, l, g)
        kb, vb = ow.block(cfg, r, l, g, x)
        cm = ow.compressed(cfg, r, l, g, kc, vc)        # cache building is not part of the round
        t0 = time.perf_counter()
        oatt.verify_unit(q, kc, vc, kb, vb)
        for i in range(x):
            oatt.draft_unit(q[i], cm.k, cm.v, kb, vb, i)
        t_units += time.perf_counter() - t0
        units += 1
    t_unit = t_units / units
    wu = np.zeros((cfg.wu_width, cfg.vocab))
    o = np.zeros((x, cfg.Hq * cfg.d))
    t0 = time.perf_counter()
    zv, zd = oacc.logits(o, wu), oacc.logits(o, wu)
    tv, _ = oacc.argmax_gap(zv)
    td, _ = oacc.argmax_gap(zd)
    oacc.accept(td, tv)
    t_inst = time.perf_counter() - t0
    n_units = cfg.B * cfg.L * cfg.Hkv
    n_inst = cfg.B * cfg.L
    round_s = t_unit * n_units + t_inst * n_inst
    return round_s, threads, (f"{units} (request, layer, kv-head) units of one round (verify pass + "
                              f"{x} draft steps; {t_units:.1f} s) and one instance's logits+accept, "
                              f"timed and scaled by {n_units} units / {n_inst} instances")


def stream_ceiling(args):
    """The box's streaming-read peak (nontemporal vector reads of a contiguous 4 GiB buffer),
    measured after the timed region; None when switched off."""
    if args.no_stream_ceiling:
        return None
    from lossless_kv_cache_vc_amd import stream_probe
    return stream_probe.measure(gib=4.0, reps=3)


def with_ceiling(roof: dict, ceiling) -> dict:
    """A roofline object plus its achieved rate as a fraction of the measured streaming-read
    peak."""
    if ceiling:
        roof["ceiling_gbps"] = ceiling["read_gbps"]
        roof["ceiling_frac"] = round(roof["achieved"] / ceiling["read_gbps"], 4)
    return roof


def bench_mixed(cfg, wl, args):
    """The ragged batch: one step is one launch over all requests, drafting and verifying."""
    import torch
    nbytes = wl.mixed_bytes()
    for _ in range(args.warmup):
        wl.run_mixed()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        wl.run_mixed()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"metric": f"mixed draft+verify attention achieved HBM TB/s ({cfg.name})",
           "value": round(gbps / 1e3, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": f"{cfg.name}: {cfg.note}", "requests": cfg.B,
                                          "parallelism": "1 GPU"},
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(args.config, "mixed"),
                        "kernel": "mixed_kernel<128>", "algorithmic_bytes_per_launch": int(nbytes)},
           "breakdown_ms": {"launch": round(ms, 4)}}
    ceiling = stream_ceiling(args)
    if ceiling:
        out["stream_ceiling"] = ceiling
        out["pct_of_stream_ceiling"] = round(100 * gbps / ceiling["read_gbps"], 2)
        with_ceiling(out["roofline"], ceiling)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip measuring the streaming-read ceiling after the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle work to time for the CPU baseline")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="0: greedy accept; > 0: drafted tokens sampled at this temperature and the "
                         "rejection-sampling accept")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: every (request, "
              "layer, kv head) unit of the path is independent, so more GPUs would each run their "
              "own share with no exchange", file=sys.stderr)
        sys.exit(2)

    import torch
    from lossless_kv_cache_vc_amd.harness import Workload
    from vcsynth import configs as C

    cfg = C.get(args.config)
    t_build = time.perf_counter()
    # growth room for committing one round's accepted rows after the timed region
    wl = Workload(cfg, spare_tokens=0 if cfg.mixed else 64)
    torch.cuda.synchronize()
    print(f"# built {cfg.name} in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)

    if cfg.mixed:
        return bench_mixed(cfg, wl, args)

    x = max(r.x for r in cfg.reqs)
    v_bytes = wl.verify_bytes()
    d_bytes = [wl.draft_bytes(i) for i in range(x)]
    round_bytes = v_bytes + sum(d_bytes)

    def one_round(evs):
        evs[0].record()
        for i in range(x):
            wl.run_draft(i)
        evs[1].record()
        wl.run_verify()
        evs[2].record()
        wl.logits()
        evs[3].record()
        wl.accept(args.temperature)
        evs[4].record()

    for _ in range(args.warmup):
        one_round([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_round(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # commit of the last round: block rows 0..a (the accepted prefix and the token before it) of
    # every request join the full and drafting caches (outside the metric; wall clock, incl. the
    # host's page-table and allocator work)
    acc = wl.acc_len.cpu().numpy()
    counts = [min(int(acc[r * cfg.L]) + 1, cfg.reqs[r].x) for r in range(cfg.B)]
    torch.cuda.synchronize()
    t_c = time.perf_counter()
    wl.commit(counts)
    torch.cuda.synchronize()
    commit_ms = (time.perf_counter() - t_c) * 1e3

    draft_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    verify_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    logits_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    accept_ms = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
    attn_ms = draft_ms + verify_ms
    value_tbs = round_bytes / (attn_ms * 1e-3) / 1e12
    ms_per_step = wall * 1e3 / args.steps

    verify_gbps = v_bytes / (verify_ms * 1e-3) / 1e9
    draft_launch_ms = draft_ms / x
    draft_gbps = (sum(d_bytes) / x) / (draft_launch_ms * 1e-3) / 1e9
    dominant = "draft" if draft_ms >= verify_ms else "verify"

    bits = cfg.reqs[0].bits
    draft_role = {16: "draft", 2: "draft_kivi2", 4: "draft_kivi4"}[bits]
    draft_name = {16: "draft_bf16_kernel<128>", 2: "draft_kivi_kernel<128, 2>", 4: "draft_kivi_kernel<128, 4>"}[bits]

    def roof(kind):
        if kind == "verify":
            # a verify-only launch of more than 128 query rows per kv head runs the wide kernel
            wide = max(r.x for r in cfg.reqs) * cfg.G > 128
            name = "verify_wide_kernel<128>" if wide else "verify_kernel<128>"
            achieved, per_launch, role = verify_gbps, v_bytes, "verify"
        else:
            achieved, per_launch, name, role = draft_gbps, sum(d_bytes) / x, draft_name, draft_role
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(args.config, role),
                "kernel": name, "algorithmic_bytes_per_launch": int(per_launch)}

    # verify MFMA use: the two bf16 products (scores and weighted values) of every query row
    # against every key it sees (the whole context plus drafted rows 0..i), 2 flops per
    # multiply-add
    v_flops = sum(4 * cfg.G * cfg.d * (r.rows * r.ctx_len + r.rows * (r.rows + 1) // 2)
                  for r in wl.verify_reqs()) * cfg.L * cfg.Hkv
    v_tflops = v_flops / (verify_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value_tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.note}",
            "batch": cfg.B, "layers": cfg.L, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
            "head_dim": cfg.d, "ctx": cfg.reqs[0].ctx_len, "x": x,
            "kept_tokens": cfg.reqs[0].kept, "parallelism": "1 GPU",
        },
        "pct_of_peak": round(100 * value_tbs * 1e3 / PEAK_HBM_GBPS, 2),
        "roofline": roof(dominant),
        "roofline_verify": roof("verify"),
        "verify_mfma": {"achieved": round(v_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(v_tflops / PEAK_BF16_TFLOPS, 4), "flops_per_launch": int(v_flops)},
        "breakdown_ms": {"draft_total": round(draft_ms, 3), "draft_per_launch": round(draft_launch_ms, 4),
                         "verify": round(verify_ms, 3), "logits": round(logits_ms, 3),
                         "accept": round(accept_ms, 4), "commit_wall": round(commit_ms, 3)},
        "committed_rows": counts,
        "accept": "greedy" if args.temperature <= 0 else f"rejection sampling, T = {args.temperature}",
        "bytes": {"verify": v_bytes, "draft_per_step_avg": int(sum(d_bytes) / x), "round": round_bytes},
    }
    ceiling = stream_ceiling(args)
    if ceiling:
        out["stream_ceiling"] = ceiling
        out["pct_of_stream_ceiling"] = round(100 * value_tbs * 1e3 / ceiling["read_gbps"], 2)
        with_ceiling(out["roofline"], ceiling)
        with_ceiling(out["roofline_verify"], ceiling)
    if not args.no_cpu_baseline:
        round_s, threads, sample = cpu_baseline(cfg, args.cpu_seconds)
        out["cpu_baseline"] = {"value": round(round_bytes / round_s / 1e12, 8), "unit": "TB/s",
                               "cores": threads, "kind": "oracle", "sample": sample,
                               "round_seconds_scaled": round(round_s, 1), "host": host_info()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
