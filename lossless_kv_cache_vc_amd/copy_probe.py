"""A plain device-to-device copy of known size, used to calibrate HBM byte counters.

rocprofv3's FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) are read for this copy and
for the attention kernels under the same conditions; the ratio of the copy's counted bytes to
its true bytes (read = written = ``--gib`` GiB) scales the attention kernels' counts.

    python -m lossless_kv_cache_vc_amd.copy_probe --gib 2 --reps 3
"""
from __future__ import annotations

import argparse
import json


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=2.0)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch
    n = int(args.gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(args.reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.reps
    nbytes = n * 4
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": args.reps,
                      "ms_per_copy": round(ms, 4), "gbps": round(2 * nbytes / ms / 1e6, 1)}))


if __name__ == "__main__":
    main()
