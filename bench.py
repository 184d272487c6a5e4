#!/usr/bin/env python3
"""Benchmark of the draft/verify attention hot path on one MI355X.

One step is one draft-verify round over the whole batch of the Llama-3.1-8B 32K workload
(8 requests, 32 layer slices, 32 query / 8 KV heads, d = 128, n = 32768, x = 32, 4x token
drop): x single-query draft launches over the compressed cache, one verify launch over the full
cache, the LM-head stand-in for both, and the greedy accept.  Inputs are resident in HBM before
the timed region.  The metric is the attention's achieved HBM bandwidth: algorithmic bytes of
the draft and verify launches divided by their measured time.

After the main line's timed region the other workloads are measured briefly (per_config): the
tiny case, 100K KIVI-2, the 128K drop + KIVI-4 workload with its full cache reloaded from pinned
host memory while the drafts run, and the 64-request ragged mixed launch.  Each reports its round
rate, the accept-length histogram and flagged-row fractions of its logits, and the oracle's
max-abs error on sampled units (from the CPU baseline leg, which runs the oracle on them).

    python bench.py [--steps K] [--warmup W] [--config C2] [--staged] [--no-cpu-baseline]
                    [--no-per-config]
"""
from __future__ import annotations

import argparse
import contextlib
import gc
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
# per-workload lines (not the headline, which keeps exactly --warmup and --steps): warm up for at
# least WARM_S seconds and time at least MIN_TIMED_S seconds, so that sub-millisecond steps are
# timed at the steady clock
WARM_S = 0.25
MIN_TIMED_S = 0.15
TIE_GAP = 1e-3  # a logits row whose top-2 gap is below this is a near-tie (flagged)


def measured_traffic(config: str, kind: str):
    """HBM bytes per launch of one attention kernel of one workload from the committed rocprofv3
    counter runs (L2-to-memory read and write requests counted by size, checked exactly on a
    device copy of known size), or None when absent or taken on other kernel code."""
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


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def _thread_limit(n):
    """Context limiting the oracle's BLAS threads to n (None: leave them)."""
    if n is None:
        return contextlib.nullcontext()
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=n)


def _context(cfg, r, l, g):
    """Context K and V rows of one (request, layer, kv head) as float64, drawn by the seeded
    generator's GPU fill kernel (bit-identical to its CPU form, and far faster at full lengths)."""
    import numpy as np
    import torch
    from vcsynth import gpu as sg
    from vcsynth import rng
    from vcsynth import tensors as T
    n = cfg.reqs[r].ctx_len
    out = []
    for stream in (rng.STREAM_KCTX, rng.STREAM_VCTX):
        t = torch.empty((n, cfg.d), dtype=torch.int16, device="cuda")
        sg.fill_normal_bf16(t, [cfg.d, 1], T.ctx_index(cfg, r, l, g, 0, 0), cfg.seed, stream)
        bits = t.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        out.append(bits.view(np.float32).astype(np.float64))
    return out[0], out[1]


def _max_err(got, want) -> float:
    import numpy as np
    return float(np.abs(np.asarray(got, dtype=np.float64) - want).max())


def cpu_baseline(cfg, wl, budget_s: float, threads=None, round_bytes=None):
    """The oracle, untuned, on a bounded sample of the same round, scaled to the whole round:
    (request, layer, kv head) units of the verify pass plus all x draft steps (or, for the ragged
    batch, whole requests of the mixed launch) are timed until about `budget_s` seconds of oracle
    work have run, plus one instance's logits and accept.  The sampled units' outputs are compared
    with the GPU's outputs of the last round (max-abs error).  threads: BLAS threads (None = all)."""
    import numpy as np
    from oracle import accept as oacc
    from oracle import attention as oatt
    from oracle import workload as ow
    from vcsynth import configs as C

    G = cfg.G
    err_v = err_d = 0.0
    with _thread_limit(threads):
        used = _blas_threads() if threads is None else threads
        t_units, units = 0.0, 0
        if cfg.mixed:
            order = sorted(range(cfg.B), key=lambda r: cfg.reqs[r].ctx_len)  # short requests first
            t_kind = {C.KIND_VERIFY: [0.0, 0], C.KIND_DRAFT: [0.0, 0]}
            for i in range(cfg.B):
                if t_units >= budget_s and all(v[1] for v in t_kind.values()):
                    break
                r = order[i // 2] if i % 2 == 0 else order[-1 - i // 2]
                req = cfg.reqs[r]
                g = r % cfg.Hkv
                xr = req.x if req.kind == C.KIND_VERIFY else req.step + 1
                q = ow.queries(cfg, r, 0, xr)[:, g * G:(g + 1) * G]
                kc, vc = _context(cfg, r, 0, g)
                kb, vb = ow.block(cfg, r, 0, g, xr)
                cm = ow.compressed(cfg, r, 0, g, kc, vc) if req.kind == C.KIND_DRAFT else None
                t0 = time.perf_counter()
                if req.kind == C.KIND_VERIFY:
                    o = oatt.verify_unit(q, kc, vc, kb, vb)
                else:
                    o = oatt.draft_unit(q[req.step], cm.k, cm.v, kb, vb, req.step)
                dt = time.perf_counter() - t0
                t_units += dt
                t_kind[req.kind][0] += dt
                t_kind[req.kind][1] += 1
                units += 1
                got = wl.out_v[r, 0, :xr, g * G:(g + 1) * G].double().cpu().numpy()
                if req.kind == C.KIND_VERIFY:
                    err_v = max(err_v, _max_err(got, o))
                else:
                    err_d = max(err_d, _max_err(got[req.step], o))
                print(f"# oracle unit {units}: request {r} ({'verify' if req.kind == C.KIND_VERIFY else 'draft'}, "
                      f"n={req.ctx_len}) {dt:.2f} s", file=sys.stderr, flush=True)
            n_ver = sum(1 for q in cfg.reqs if q.kind == C.KIND_VERIFY)
            per = {k: v[0] / max(1, v[1]) for k, v in t_kind.items()}
            round_s = cfg.Hkv * (per[C.KIND_VERIFY] * n_ver + per[C.KIND_DRAFT] * (cfg.B - n_ver))
            sample = (f"{units} (request, kv head) units of the mixed launch ({t_units:.1f} s), "
                      f"scaled by {cfg.Hkv} kv heads per request and the verify / draft mix")
        else:
            x = cfg.reqs[0].x
            while t_units < budget_s and units < cfg.B * cfg.L * cfg.Hkv:
                r, l, g = units % cfg.B, (7 * units) % cfg.L, (3 * units) % cfg.Hkv
                q = ow.queries(cfg, r, l, x)[:, g * G:(g + 1) * G]
                kc, vc = _context(cfg, r, l, g)
                kb, vb = ow.block(cfg, r, l, g, x)
                cm = ow.compressed(cfg, r, l, g, kc, vc)        # cache building is not part of the round
                t0 = time.perf_counter()
                ver = oatt.verify_unit(q, kc, vc, kb, vb)
                dr = [oatt.draft_unit(q[i], cm.k, cm.v, kb, vb, i) for i in range(x)]
                t_units += time.perf_counter() - t0
                units += 1
                sl = slice(g * G, (g + 1) * G)
                err_v = max(err_v, _max_err(wl.out_v[r, l, :x, sl].double().cpu().numpy(), ver))
                err_d = max(err_d, _max_err(wl.out_d[r, l, :x, sl].double().cpu().numpy(), np.stack(dr)))
                print(f"# oracle unit {units} (r={r}, l={l}, g={g}): {t_units:.1f} s of oracle work so far",
                      file=sys.stderr, flush=True)
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
            sample = (f"{units} (request, layer, kv-head) units of one round (verify pass + {x} draft "
                      f"steps; {t_units:.1f} s) and one instance's logits+accept, timed and scaled by "
                      f"{n_units} units / {n_inst} instances")
    out = {"value": None, "unit": "TB/s", "cores": used, "kind": "oracle", "sample": sample,
           "round_seconds_scaled": round(round_s, 2),
           "max_abs_err_vs_gpu": {"verify": float(f"{err_v:.3e}"), "draft": float(f"{err_d:.3e}"),
                                  "units": units}}
    if round_bytes:
        out["value"] = round(round_bytes / round_s / 1e12, 8)
    return out


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


def logits_evidence(cfg, wl):
    """Near-tie rows (top-2 logit gap below 1e-3 in the GPU's own logits) of the draft and verify
    rows that belong to the round, and the histogram of accept lengths over every instance."""
    import torch
    B, L, xm = cfg.B, cfg.L, wl.xmax
    V = cfg.vocab

    def flagged(z):
        top2 = torch.topk(z.view(B * L, xm, V), 2, dim=-1).values
        gap = (top2[..., 0] - top2[..., 1]).cpu()
        rows = torch.zeros(B * L, xm, dtype=torch.bool)
        for r in range(B):
            rr = range(cfg.reqs[r].x) if not cfg.mixed else (
                range(cfg.reqs[r].x) if cfg.reqs[r].kind == 0 else [cfg.reqs[r].step])
            for l in range(L):
                rows[r * L + l, list(rr)] = True
        return round(float((gap[rows] < TIE_GAP).float().mean()), 4), int(rows.sum())

    fv, nv = flagged(wl.z_v)
    out = {"flagged_rows": {"verify": fv, "rows_verify": nv}}
    if not cfg.mixed:
        fd, nd = flagged(wl.z_d)
        out["flagged_rows"].update({"draft": fd, "rows_draft": nd})
        acc = wl.acc_len.cpu().tolist()
        hist = {}
        for a in acc:
            hist[str(a)] = hist.get(str(a), 0) + 1
        out["accept_len_hist"] = dict(sorted(hist.items(), key=lambda kv: int(kv[0])))
        out["accept_len_mean"] = round(sum(acc) / len(acc), 3)
    return out


def warm_up(step, warmup, warm_s):
    """`warmup` untimed steps, then more until `warm_s` seconds of wall time have passed; returns
    (steps run, wall seconds per step).  After an idle gap the GPU clock climbs for some tens of
    milliseconds, so a workload whose step is a fraction of a millisecond, timed right after a
    couple of warm-up steps, reads the climb rather than the steady rate."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < warmup or (warm_s > 0 and time.perf_counter() - t0 < warm_s):
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()  # keep the host within a few steps of the GPU
    torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) / max(n, 1)


def timed_steps(steps, per_step_s, min_timed_s, cap=4000):
    """At least `steps`, and enough that the timed region spans `min_timed_s` seconds."""
    if min_timed_s <= 0 or per_step_s <= 0:
        return steps
    return max(steps, min(cap, int(min_timed_s / per_step_s) + 1))


def time_round(cfg, wl, steps, warmup, temperature=0.0, warm_s=0.0, min_timed_s=0.0):
    """Warm-up rounds, then `steps` timed rounds (more with `min_timed_s`); per-phase
    milliseconds from HIP events on the stream the kernels run on."""
    import torch
    x = max(r.x for r in cfg.reqs)

    def one_round(evs):
        evs[0].record()
        for i in range(x):
            wl.run_draft(i)
        evs[1].record()
        wl.run_verify()
        evs[2].record()
        wl.logits()
        evs[3].record()
        wl.accept(temperature)
        evs[4].record()

    warmed, per_round = warm_up(lambda: one_round([torch.cuda.Event(enable_timing=True) for _ in range(5)]),
                                warmup, warm_s)
    steps = timed_steps(steps, per_round, min_timed_s)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one_round(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / steps
    return {"draft": ms(0, 1), "verify": ms(1, 2), "logits": ms(2, 3), "accept": ms(3, 4),
            "wall_ms_per_step": wall * 1e3 / steps, "steps": steps, "warmup": warmed}


def round_record(cfg, wl, t, steps, warmup):
    """Rates and rooflines of a timed round (no oracle)."""
    x = max(r.x for r in cfg.reqs)
    v_bytes = wl.verify_bytes()
    d_bytes = [wl.draft_bytes(i) for i in range(x)]
    round_bytes = v_bytes + sum(d_bytes)
    attn_ms = t["draft"] + t["verify"]
    value_tbs = round_bytes / (attn_ms * 1e-3) / 1e12
    verify_gbps = v_bytes / (t["verify"] * 1e-3) / 1e9
    draft_launch_ms = t["draft"] / x
    draft_gbps = (sum(d_bytes) / x) / (draft_launch_ms * 1e-3) / 1e9
    bits = cfg.reqs[0].bits
    draft_role = {16: "draft", 2: "draft_kivi2", 4: "draft_kivi4"}[bits]
    draft_name = {16: "draft_bf16_kernel<128>", 2: "draft_kivi_kernel<128, 2>",
                  4: "draft_kivi_kernel<128, 4>"}[bits]
    key = cfg.name.split("-")[0]

    def roof(kind):
        if kind == "verify":
            # a verify-only launch of more than 128 query rows per kv head runs the wide kernel
            wide = x * cfg.G > 128
            name = "verify_wide_kernel<128>" if wide else "verify_kernel<128>"
            achieved, per_launch, role = verify_gbps, v_bytes, "verify"
        else:
            achieved, per_launch, name, role = draft_gbps, sum(d_bytes) / x, draft_name, draft_role
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(key, role),
                "kernel": name, "algorithmic_bytes_per_launch": int(per_launch)}

    # verify MFMA use: the two bf16 products (scores and weighted values) of every query row
    # against every key it sees (the whole context plus drafted rows 0..i), 2 flops per
    # multiply-add
    v_flops = sum(4 * cfg.G * cfg.d * (r.rows * r.ctx_len + r.rows * (r.rows + 1) // 2)
                  for r in wl.verify_reqs()) * cfg.L * cfg.Hkv
    v_tflops = v_flops / (t["verify"] * 1e-3) / 1e12
    dominant = "draft" if t["draft"] >= t["verify"] else "verify"
    return {
        "value": round(value_tbs, 4),
        "ms_per_step": round(t["wall_ms_per_step"], 3),
        "roofline": roof(dominant),
        "roofline_verify": roof("verify"),
        "roofline_draft": roof("draft"),
        "verify_mfma": {"achieved": round(v_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(v_tflops / PEAK_BF16_TFLOPS, 4), "flops_per_launch": int(v_flops)},
        "breakdown_ms": {"draft_total": round(t["draft"], 3), "draft_per_launch": round(draft_launch_ms, 4),
                         "verify": round(t["verify"], 3), "logits": round(t["logits"], 3),
                         "accept": round(t["accept"], 4)},
        "bytes": {"verify": v_bytes, "draft_per_step_avg": int(sum(d_bytes) / x), "round": round_bytes},
        "steps": steps, "warmup": warmup,
    }


def staged_round(cfg, wl, steps, draft_ms_alone=None):
    """The full cache in pinned host memory, reloaded into HBM while the drafter runs: per round,
    every layer slice of the full pool is copied from exact-size pinned host buffers by
    vc_stage_kv on a side stream while the x draft launches run on the compute stream; the
    compute stream waits on the staging event and runs the verify.  The pool is cleared before
    the first reload, so every verify reads staged bytes."""
    import torch
    x = max(r.x for r in cfg.reqs)
    t0 = time.perf_counter()
    bufs = wl.full_to_host()
    setup_s = time.perf_counter() - t0
    wl.full.k.zero_()
    wl.full.v.zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    recs = []
    for _ in range(steps):
        st0 = torch.cuda.Event(enable_timing=True)
        staged = torch.cuda.Event(enable_timing=True)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        st0.record(side)
        e[0].record()
        nbytes = wl.stage_full(bufs, side, staged)
        for i in range(x):
            wl.run_draft(i)
        e[1].record()
        torch.cuda.current_stream().wait_event(staged)
        e[2].record()
        wl.run_verify()
        e[3].record()
        torch.cuda.synchronize()
        recs.append({"stage_ms": st0.elapsed_time(staged), "draft_ms": e[0].elapsed_time(e[1]),
                     "round_ms": e[0].elapsed_time(e[3]), "verify_ms": e[2].elapsed_time(e[3]),
                     "bytes": nbytes})
    del bufs
    avg = lambda k: sum(r[k] for r in recs) / len(recs)
    nbytes = recs[0]["bytes"]
    return {"staged_bytes": nbytes, "stage_gbps": round(nbytes / (avg("stage_ms") * 1e-3) / 1e9, 2),
            "stage_ms": round(avg("stage_ms"), 2),
            "draft_ms_per_launch_during_copy": round(avg("draft_ms") / x, 4),
            "draft_ms_per_launch_alone": None if draft_ms_alone is None else round(draft_ms_alone / x, 4),
            "verify_ms_after_wait": round(avg("verify_ms"), 3), "round_ms": round(avg("round_ms"), 2),
            "drafts_inside_copy_window": bool(all(r["draft_ms"] <= r["stage_ms"] for r in recs)),
            "pinned_setup_s": round(setup_s, 1), "rounds": len(recs),
            "note": "full pool cleared first; the verify reads only staged bytes"}


def mixed_record(cfg, wl, steps, warmup, warm_s=0.0, min_timed_s=0.0):
    import torch
    nbytes = wl.mixed_bytes()
    warmup, per_launch = warm_up(wl.run_mixed, warmup, warm_s)
    steps = timed_steps(steps, per_launch, min_timed_s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        wl.run_mixed()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"value": round(gbps / 1e3, 4), "ms_per_step": round(wall * 1e3 / steps, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("C5", "mixed"),
                         "kernel": "mixed_kernel<128>", "algorithmic_bytes_per_launch": int(nbytes)},
            "breakdown_ms": {"launch": round(ms, 4)}, "steps": steps, "warmup": warmup,
            "bytes": {"launch": nbytes}}


def measure_config(name, steps, warmup, cpu_budget, staged=False, temperature=0.0):
    """One workload: build, time, evidence, and the oracle on sampled units (errors)."""
    import torch
    from lossless_kv_cache_vc_amd.harness import Workload
    from vcsynth import configs as C
    cfg = C.get(name)
    t_build = time.perf_counter()
    wl = Workload(cfg)
    torch.cuda.synchronize()
    print(f"# built {cfg.name} in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)
    rec = {"workload": f"{cfg.name}: {cfg.note}"}
    if cfg.mixed:
        rec.update(mixed_record(cfg, wl, steps, warmup, warm_s=WARM_S, min_timed_s=MIN_TIMED_S))
        wl.logits()
        rec.update(logits_evidence(cfg, wl))
        round_bytes = rec["bytes"]["launch"]
    else:
        t = time_round(cfg, wl, steps, warmup, temperature, warm_s=WARM_S, min_timed_s=MIN_TIMED_S)
        rec.update(round_record(cfg, wl, t, t["steps"], t["warmup"]))
        rec.update(logits_evidence(cfg, wl))
        round_bytes = rec["bytes"]["round"]
    if cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(cfg, wl, cpu_budget, round_bytes=round_bytes)
    if staged:
        rec["staged"] = staged_round(cfg, wl, max(2, min(steps, 3)),
                                     draft_ms_alone=None if cfg.mixed else rec["breakdown_ms"]["draft_total"])
    del wl
    gc.collect()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--staged", action="store_true",
                    help="also reload the full cache from pinned host memory during the drafts "
                         "(the 128K drop + KIVI-4 workload does this in per_config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the short measurements of the other workloads after the main line's")
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

    out = {"metric": METRIC if args.config == "C2" and not cfg.mixed else
           f"verify+draft attention achieved HBM TB/s ({cfg.name})"}
    if cfg.mixed:
        rec = mixed_record(cfg, wl, args.steps, args.warmup)
        out["metric"] = f"mixed draft+verify attention achieved HBM TB/s ({cfg.name})"
        wl.logits()
        ev = logits_evidence(cfg, wl)
        round_bytes = rec["bytes"]["launch"]
    else:
        t = time_round(cfg, wl, args.steps, args.warmup, args.temperature)
        rec = round_record(cfg, wl, t, args.steps, args.warmup)
        ev = logits_evidence(cfg, wl)
        round_bytes = rec["bytes"]["round"]
    out.update({
        "value": rec["value"], "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "batch": cfg.B, "layers": cfg.L,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.d,
                   "ctx": cfg.reqs[0].ctx_len, "x": max(r.x for r in cfg.reqs),
                   "kept_tokens": cfg.reqs[0].kept, "parallelism": "1 GPU"},
        "pct_of_peak": round(100 * rec["value"] * 1e3 / PEAK_HBM_GBPS, 2),
    })
    for k in ("roofline", "roofline_verify", "roofline_draft", "verify_mfma", "breakdown_ms", "bytes"):
        if k in rec:
            out[k] = rec[k]
    out["step_time_note"] = ("ms_per_step is the host wall clock of a whole round: the draft and verify "
                             "launches plus the LM-head stand-in and the accept (breakdown_ms.logits, "
                             ".accept); value counts the attention launches only")
    out.update(ev)
    out["accept"] = "greedy" if args.temperature <= 0 else f"rejection sampling, T = {args.temperature}"

    if not cfg.mixed:
        # commit of the last round: block rows 0..a (the accepted prefix and the token before it) of
        # every request join the full and drafting caches (outside the metric; wall clock, incl.
        # the host's page-table and allocator work)
        acc = wl.acc_len.cpu().numpy()
        counts = [min(int(acc[r * cfg.L]) + 1, cfg.reqs[r].x) for r in range(cfg.B)]
        torch.cuda.synchronize()
        t_c = time.perf_counter()
        wl.commit(counts)
        torch.cuda.synchronize()
        out["breakdown_ms"]["commit_wall"] = round((time.perf_counter() - t_c) * 1e3, 3)
        out["committed_rows"] = counts

    print(f"# timed {args.steps} rounds of {cfg.name}: {rec['value']} TB/s", file=sys.stderr, flush=True)
    ceiling = stream_ceiling(args)
    if ceiling:
        out["stream_ceiling"] = ceiling
        out["pct_of_stream_ceiling"] = round(100 * rec["value"] * 1e3 / ceiling["read_gbps"], 2)
        for k in ("roofline", "roofline_verify", "roofline_draft"):
            if k in out:
                with_ceiling(out[k], ceiling)
    if not args.no_cpu_baseline:
        # the oracle on the host's cores and on one core; the round's GPU outputs were overwritten by
        # the commit's next-round state only in the caches, not in out_v / out_d
        out["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_seconds, round_bytes=round_bytes)
        out["cpu_baseline"]["host"] = host_info()
        out["cpu_baseline_1core"] = cpu_baseline(cfg, wl, args.cpu_seconds / 3, threads=1,
                                                 round_bytes=round_bytes)
    if args.staged and not cfg.mixed:
        out["staged"] = staged_round(cfg, wl, 3, draft_ms_alone=out["breakdown_ms"]["draft_total"])
    del wl
    gc.collect()
    torch.cuda.empty_cache()

    if not args.no_per_config:
        per = {}
        for name in ("C1", "C3", "C4", "C5"):
            if name == args.config:
                continue
            try:
                per[name] = measure_config(name, steps=3, warmup=1,
                                           cpu_budget=0 if args.no_cpu_baseline else 3.0,
                                           staged=(name == "C4"))
            except Exception as e:  # noqa: BLE001 -- keep the main line; say what failed
                per[name] = {"error": f"{type(e).__name__}: {e}"}
                gc.collect()
                torch.cuda.empty_cache()
            print(f"# measured {name}", file=sys.stderr, flush=True)
        out["per_config"] = per
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
