"""Turn rocprofv3 output into the short summaries kept under ``profiles/``.

Measurement tooling only (it reads CSV files; it launches nothing on the GPU).

* ``stats``   — per-kernel average duration from ``--kernel-trace --stats -f csv`` output.
* ``traffic`` — HBM bytes per launch of the attention kernels of one workload from two ``--pmc``
  runs (``FETCH_SIZE``, then ``WRITE_SIZE``, KiB per dispatch), each scaled by what the same
  counter reads for a plain device copy of known size (``copy_probe.py``).  The result is merged
  into a JSON file (one entry per workload) together with a hash of the attention source, so a
  later change to the kernels makes the stored traffic stale (the benchmark then reports
  ``null``).
* ``sq``      — instruction and MFMA counters of the verify kernel (utilisation figures).

    python -m lossless_kv_cache_vc_amd.profiling stats --csv DIR/x_kernel_stats.csv --out profiles/a.md --cmd "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN_SRC = os.path.join(PKG, "csrc", "vc_attn.hip")

# kernel-name fragment -> role reported by the benchmark
ROLES = {
    "verify_kernel<128>": "verify",
    "verify_wide_kernel<128>": "verify",
    "draft_bf16_kernel<128>": "draft",
    "draft_kivi_kernel<128, 2>": "draft_kivi2",
    "draft_kivi_kernel<128, 4>": "draft_kivi4",
    "mixed_kernel<128>": "mixed",
    "merge_kernel<128>": "merge",
}


def attn_source_hash() -> str:
    """Short hash of the attention kernels' source (stored traffic is valid only for it)."""
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _role(name: str):
    for frag, role in ROLES.items():
        if frag in name:
            return role
    return None


def _counters(path_glob: str) -> Dict[str, Dict[str, List[float]]]:
    out: Dict[str, Dict[str, List[float]]] = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in sorted(glob.glob(path_glob)):
        with open(path) as f:
            for r in csv.DictReader(f):
                out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def _avg(v: List[float]) -> float:
    return sum(v) / len(v) if v else 0.0


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("vc::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        name = name.replace("void ", "").split("(")[0]
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(args):
    fetch = _counters(os.path.join(args.fetch, "*counter_collection.csv"))
    write = _counters(os.path.join(args.write, "*counter_collection.csv"))
    cf = _counters(os.path.join(args.copy_fetch, "*counter_collection.csv"))
    cw = _counters(os.path.join(args.copy_write, "*counter_collection.csv"))

    def copy_kib(c, counter):
        vals = [v for name, d in c.items() if "copyBuffer" in name or "elementwise" in name
                for v in d.get(counter, []) if v > 1024]
        return max(vals) if vals else 0.0

    true_kib = args.copy_bytes / 1024.0
    f_fetch = true_kib / copy_kib(cf, "FETCH_SIZE")
    f_write = true_kib / copy_kib(cw, "WRITE_SIZE")
    try:
        rec = json.load(open(args.json))
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_hash") != attn_source_hash():
        rec = {}
    rec.update({"source_hash": attn_source_hash(), "fetch_scale": round(f_fetch, 4),
                "write_scale": round(f_write, 4), "copy_bytes": args.copy_bytes})
    rec.setdefault("configs", {})
    entry = {"command": args.cmd, "kernels": {}}
    rec["configs"][args.config] = entry
    lines = [f"# {args.title}", "", "Commands (one counter per run, then the same for the copy probe):", "",
             "```", args.cmd, "```", "",
             f"Copy calibration ({args.copy_bytes / 2**30:.0f} GiB device copy): FETCH_SIZE reads "
             f"{copy_kib(cf, 'FETCH_SIZE'):.0f} KiB, WRITE_SIZE {copy_kib(cw, 'WRITE_SIZE'):.0f} KiB for "
             f"{true_kib:.0f} KiB moved each way; scale factors {f_fetch:.3f} (fetch), {f_write:.3f} (write).",
             "", "| kernel | launches | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | HBM bytes/launch (scaled) |",
             "|---|---|---|---|---|"]
    for name in sorted(set(fetch) | set(write)):
        role = _role(name)
        if role is None:
            continue
        fk, wk = _avg(fetch[name].get("FETCH_SIZE", [])), _avg(write[name].get("WRITE_SIZE", []))
        b = fk * 1024 * f_fetch + wk * 1024 * f_write
        entry["kernels"][role] = {"bytes_per_launch": int(b), "fetch_kib": fk, "write_kib": wk,
                                  "launches": len(fetch[name].get("FETCH_SIZE", []))}
        lines.append(f"| {role} | {len(fetch[name].get('FETCH_SIZE', []))} | {fk:.0f} | {wk:.0f} | {b:.4g} |")
    if args.note:
        lines += ["", args.note]
    json.dump(rec, open(args.json, "w"), indent=1)
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _req_bytes(reads: Dict[str, List[float]], writes: Dict[str, List[float]]):
    """Read and write bytes per dispatch from the request-size counters: each read request is 32,
    64 or 128 bytes (TCC_EA0_RDREQ_32B/_64B/_128B), each write 32 or 64 bytes (TCC_EA0_WRREQ minus
    TCC_EA0_WRREQ_64B, and TCC_EA0_WRREQ_64B); lists are per dispatch."""
    n32, n64, n128 = (reads.get(f"TCC_EA0_RDREQ_{k}_sum", []) for k in ("32B", "64B", "128B"))
    tot = reads.get("TCC_EA0_RDREQ_sum", [])
    wr, w64 = writes.get("TCC_EA0_WRREQ_sum", []), writes.get("TCC_EA0_WRREQ_64B_sum", [])
    rd_b = [32 * a + 64 * b + 128 * c for a, b, c in zip(n32, n64, n128)]
    wr_b = [32 * (a - b) + 64 * b for a, b in zip(wr, w64)]
    unsized = [t - (a + b + c) for t, a, b, c in zip(tot, n32, n64, n128)]
    return rd_b, wr_b, unsized


def cmd_traffic_req(args):
    """HBM bytes per launch from request-size counters (no fitted scale): the copy probe's counted
    bytes are compared with its true bytes as a check of the counters, not used as a factor."""
    reads = _counters(os.path.join(args.reads, "*counter_collection.csv"))
    writes = _counters(os.path.join(args.writes, "*counter_collection.csv"))
    creads = _counters(os.path.join(args.copy_reads, "*counter_collection.csv"))
    cwrites = _counters(os.path.join(args.copy_writes, "*counter_collection.csv"))
    # the copy is the dispatch that reads the most (the probe also runs a fill first)
    copy_name = max(creads, key=lambda n: max(creads[n].get("TCC_EA0_RDREQ_sum", [0.0])), default=None)
    cr, cw, cu = _req_bytes(creads.get(copy_name, {}), cwrites.get(copy_name, {}))
    copy_read = max(cr) if cr else 0.0
    copy_write = max(cw) if cw else 0.0
    check_r = copy_read / args.copy_bytes if args.copy_bytes else None
    check_w = copy_write / args.copy_bytes if args.copy_bytes else None
    try:
        rec = json.load(open(args.json))
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_hash") != attn_source_hash():
        rec = {}
    rec.update({"source_hash": attn_source_hash(), "method": "request-size counters (32/64/128-byte reads, "
                "32/64-byte writes)", "copy_bytes": args.copy_bytes,
                "copy_check": {"read_ratio": None if check_r is None else round(check_r, 4),
                               "write_ratio": None if check_w is None else round(check_w, 4)}})
    rec.setdefault("configs", {})
    entry = {"command": args.cmd, "kernels": {}}
    rec["configs"][args.config] = entry
    lines = [f"# {args.title}", "", "Commands (request-size counters; reads and writes in separate runs, then the "
             "same for the copy probe):", "", "```", args.cmd, "```", "",
             f"Bytes = 32 x TCC_EA0_RDREQ_32B + 64 x TCC_EA0_RDREQ_64B + 128 x TCC_EA0_RDREQ_128B (reads) and "
             f"32 x (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) + 64 x TCC_EA0_WRREQ_64B (writes), summed over the L2 "
             f"channels, per dispatch.  Check on a {args.copy_bytes / 2**30:.0f} GiB device copy: "
             f"{copy_read / 2**30:.4f} GiB read and {copy_write / 2**30:.4f} GiB written by these counters "
             f"(ratios {check_r:.4f} and {check_w:.4f}); requests the size counters do not classify: "
             f"{int(max(cu) if cu else 0)}.", "",
             "| kernel | launches | read bytes/launch | write bytes/launch | HBM bytes/launch | unsized read requests |",
             "|---|---|---|---|---|---|"]
    for name in sorted(set(reads) | set(writes)):
        role = _role(name)
        if role is None:
            continue
        rb, wb, un = _req_bytes(reads[name], writes.get(name, {}))
        r, w = _avg(rb), _avg(wb)
        entry["kernels"][role] = {"bytes_per_launch": int(r + w), "read_bytes": int(r), "write_bytes": int(w),
                                  "launches": len(rb), "unsized_read_requests": _avg(un)}
        lines.append(f"| {role} | {len(rb)} | {r:.4g} | {w:.4g} | {r + w:.4g} | {_avg(un):.0f} |")
    if args.note:
        lines += ["", args.note]
    json.dump(rec, open(args.json, "w"), indent=1)
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_sq(args):
    c = _counters(os.path.join(args.dir, "*", "*counter_collection.csv"))
    lines = [f"# {args.title}", "", "Commands:", "", "```", args.cmd, "```", "",
             "| kernel | counter | avg per launch |", "|---|---|---|"]
    for name, d in sorted(c.items()):
        role = _role(name)
        if role is None:
            continue
        for counter, vals in sorted(d.items()):
            lines.append(f"| {role} | {counter} | {_avg(vals):.4g} |")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="Kernel trace summary")
    s.add_argument("--cmd", required=True)
    s.add_argument("--note", default="")
    s.set_defaults(fn=cmd_stats)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--config", required=True, help="workload id the counters were taken on (e.g. C2)")
    t.add_argument("--json", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="HBM traffic per launch")
    t.add_argument("--cmd", required=True)
    t.add_argument("--note", default="")
    t.set_defaults(fn=cmd_traffic)
    r = sub.add_parser("traffic-req")
    for k in ("reads", "writes", "copy_reads", "copy_writes"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--config", required=True, help="workload id the counters were taken on (e.g. C2)")
    r.add_argument("--json", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--title", default="HBM traffic per launch")
    r.add_argument("--cmd", required=True)
    r.add_argument("--note", default="")
    r.set_defaults(fn=cmd_traffic_req)
    q = sub.add_parser("sq")
    q.add_argument("--dir", required=True)
    q.add_argument("--out", required=True)
    q.add_argument("--title", default="SQ counters")
    q.add_argument("--cmd", required=True)
    q.add_argument("--note", default="")
    q.set_defaults(fn=cmd_sq)
    args = ap.parse_args()
    args.fn(args)


if __name__ == "__main__":
    main()
