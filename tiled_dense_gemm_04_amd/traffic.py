"""HBM-side traffic of a GEMM launch from rocprofv3 counter runs.

Reads four rocprofv3 ``--pmc`` CSV outputs (``*_counter_collection.csv``): FETCH_SIZE and
WRITE_SIZE of a plain device copy of a known byte count, and the same two counters for
the GEMM. Each GEMM counter is scaled by (known bytes / counter value of the copy), so the
result is in bytes moved between the L2s and the memory side (Infinity Cache + HBM) per
launch. Writes profiles/traffic_<config>_<workload>.json (read by bench.py when the kernel
source hash matches) and prints a short summary.

  python -m tiled_dense_gemm_04_amd.traffic --copy-fetch DIR --copy-write DIR \\
      --gemm-fetch DIR --gemm-write DIR --copy-bytes 268435456 --config NAME --workload NAME
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def per_dispatch_kib(run_dir: str, name_filter: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "*counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    sums = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_filter not in r["Kernel_Name"] or r["Counter_Name"] != counter:
                    continue
                key = (f, int(r["Dispatch_Id"]))
                sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
    return [sums[k] for k in sorted(sums)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--gemm-fetch", required=True)
    ap.add_argument("--gemm-write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--config", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()

    from bench import kernel_source_hash

    known_kib = args.copy_bytes / 1024.0
    # the copy runs as the runtime's blit kernel (torch's elementwise kernel is the fill)
    cf = [v for v in per_dispatch_kib(args.copy_fetch, "copyBuffer", "FETCH_SIZE") if v > 0.1 * known_kib]
    cw = [v for v in per_dispatch_kib(args.copy_write, "copyBuffer", "WRITE_SIZE") if v > 0.1 * known_kib]
    gf = per_dispatch_kib(args.gemm_fetch, "gemm", "FETCH_SIZE")
    gw = per_dispatch_kib(args.gemm_write, "gemm", "WRITE_SIZE")
    f_scale = known_kib / statistics.median(cf)
    w_scale = known_kib / statistics.median(cw)
    fetch = statistics.median(gf) * f_scale * 1024
    write = statistics.median(gw) * w_scale * 1024
    out = {
        "config": args.config,
        "workload": args.workload,
        "kernel_source_hash": kernel_source_hash(),
        "copy_bytes": args.copy_bytes,
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "fetch_bytes_per_launch": int(fetch),
        "write_bytes_per_launch": int(write),
        "hbm_bytes_per_launch": int(fetch + write),
        "dispatches": {"gemm_fetch": len(gf), "gemm_write": len(gw)},
    }
    os.makedirs(args.out_dir, exist_ok=True)
    path = os.path.join(args.out_dir, f"traffic_{args.config}_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
