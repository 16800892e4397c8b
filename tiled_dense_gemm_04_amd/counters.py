"""Hardware counters of each workload's GEMM kernel, one rocprofv3 pass per counter group.

Runs (as child processes; this process never touches the GPU and never loads the HIP
library):
  * a plain 256 MiB device copy (bench.py --copy-probe) under FETCH_SIZE and under
    WRITE_SIZE: the known byte count calibrates both counters;
  * for every workload, bench.py (default config, 1 warm-up + 3 timed calls, no CPU
    baseline) under three passes:
      SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS
          SQ_INSTS_MFMA GRBM_GUI_ACTIVE
      FETCH_SIZE
      WRITE_SIZE
Each pass runs as `timeout -s KILL 60 rocprofv3 --pmc ... --output-format csv -d DIR -o p
-- python3 bench.py ...` from /tmp. The first pass that fails stops the run.

Derived per launch (median over the GEMM dispatches):
  MFMA busy      = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs)
  bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles lost per LDS cycle)
  HBM-side bytes = FETCH_SIZE * fetch scale + WRITE_SIZE * write scale (scales from the copy)
Writes profiles/traffic_<config>_<workload>.json (bench.py reports `roofline.traffic`
from it while the kernel sources still hash the same) and a markdown summary.

  python -m tiled_dense_gemm_04_amd.counters --out-dir OUT/counters \\
      [--workloads a,b] [--md profiles/counters_all_workloads.md] [--measure-json m.json]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tiled_dense_gemm_04_amd.traffic import per_dispatch_kib  # noqa: E402

COPY_BYTES = 256 << 20
SQ_SET = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
          "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"]
NUM_SIMD = 1024
NUM_XCD = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rocprof_pass(counters, out_dir, bench_args):
    """One counter pass; returns the output directory. Raises on failure."""
    os.makedirs(out_dir, exist_ok=True)
    cmd = ["timeout", "-s", "KILL", "60", "rocprofv3", "--pmc", *counters, "--output-format", "csv",
           "-d", out_dir, "-o", "p", "--", sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    log("pass:", " ".join(cmd))
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(out_dir.rstrip("/") + ".log", "w") as f:
        f.write(r.stdout + r.stderr)
    have_csv = any(n.endswith("counter_collection.csv") for _, _, fs in os.walk(out_dir) for n in fs)
    # rocprofv3 may itself end with SIGSEGV after the profiled program finished and its
    # results were written; anything else (or missing results) is a failure.
    if r.returncode != 0 and not (r.returncode in (139, -11) and have_csv):
        raise RuntimeError(f"rocprofv3 pass failed with status {r.returncode}; see {out_dir}.log")
    if not have_csv:
        raise RuntimeError(f"rocprofv3 pass wrote no counter CSV; see {out_dir}.log")
    return out_dir, r.stdout


def bench_line(stdout):
    """The JSON line bench.py printed."""
    for line in reversed(stdout.splitlines()):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise RuntimeError("bench.py printed no result line")


def sub_dir(base, name):
    return os.path.join(base, name)


def median_counter(run_dir, kernel_filter, counter):
    vals = per_dispatch_kib(run_dir, kernel_filter, counter)
    if not vals:
        raise RuntimeError(f"no {counter} values for kernels matching {kernel_filter!r} in {run_dir}")
    return statistics.median(vals)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out-dir", required=True)
    ap.add_argument("--workloads", default=None)
    ap.add_argument("--md", default=None)
    ap.add_argument("--measure-json", default=None, help="measure.py output: adds GB/s at the hot time")
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()

    import tgemm_workloads as W
    from bench import kernel_source_hash

    works = W.all_workloads() + [fw for fw in W.FP8_WORKLOADS.values() if not fw.linear]
    if args.workloads:
        keep = set(args.workloads.split(","))
        works = [w for w in works if w.name in keep]
    hot = {}
    if args.measure_json:
        with open(args.measure_json) as f:
            mj = json.load(f)
            for r in mj["results"] + (mj.get("fp8") or []):
                hot[r["workload"]] = r["hot"]["median_us"]

    out = os.path.abspath(args.out_dir)  # the passes run from /tmp
    copy_args = ["--copy-probe", str(COPY_BYTES)]
    cf, _ = rocprof_pass(["FETCH_SIZE"], sub_dir(out, "copy_FETCH_SIZE"), copy_args)
    cw, _ = rocprof_pass(["WRITE_SIZE"], sub_dir(out, "copy_WRITE_SIZE"), copy_args)
    known_kib = COPY_BYTES / 1024.0
    f_vals = [v for v in per_dispatch_kib(cf, "copyBuffer", "FETCH_SIZE") if v > 0.1 * known_kib]
    w_vals = [v for v in per_dispatch_kib(cw, "copyBuffer", "WRITE_SIZE") if v > 0.1 * known_kib]
    if not f_vals or not w_vals:
        raise RuntimeError("copy calibration found no copy dispatch")
    f_scale = known_kib / statistics.median(f_vals)
    w_scale = known_kib / statistics.median(w_vals)
    log(f"calibration: FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}")

    src_hash = kernel_source_hash()
    rows = []
    for w in works:
        bargs = ["--workload", w.name, "--steps", "3", "--warmup", "1", "--no-cpu-baseline"]
        d_sq, so = rocprof_pass(SQ_SET, sub_dir(out, f"{w.name}_sq"), bargs)
        name = bench_line(so)["config"]["kernel_config"]
        d_f, _ = rocprof_pass(["FETCH_SIZE"], sub_dir(out, f"{w.name}_FETCH_SIZE"), bargs)
        d_w, _ = rocprof_pass(["WRITE_SIZE"], sub_dir(out, f"{w.name}_WRITE_SIZE"), bargs)
        c = {k: median_counter(d_sq, "gemm", k) for k in SQ_SET}
        fetch = median_counter(d_f, "gemm", "FETCH_SIZE") * f_scale * 1024
        write = median_counter(d_w, "gemm", "WRITE_SIZE") * w_scale * 1024
        cycles = c["GRBM_GUI_ACTIVE"] / NUM_XCD
        comp = getattr(w, "compulsory_bytes", 2 * (w.M * w.K + w.K * w.N + w.M * w.N))
        row = {
            "workload": w.name, "config": name, "kernel_source_hash": src_hash,
            "mfma_busy_pct": 100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(cycles * NUM_SIMD, 1),
            "lds_bank_conflict_pct": 100 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1),
            "lds_insts": c["SQ_INSTS_LDS"], "mfma_insts": c["SQ_INSTS_MFMA"],
            "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
            "hbm_bytes_per_launch": int(fetch + write), "compulsory_bytes": comp,
            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "copy_bytes": COPY_BYTES,
        }
        if w.name in hot:
            row["hbm_gbps_at_hot_time"] = (fetch + write) / (hot[w.name] * 1e-6) / 1e9
        rows.append(row)
        os.makedirs(args.profiles, exist_ok=True)
        with open(os.path.join(args.profiles, f"traffic_{name}_{w.name}.json"), "w") as f:
            json.dump({"config": name, "workload": w.name, "kernel_source_hash": src_hash,
                       "copy_bytes": COPY_BYTES, "fetch_scale": row["fetch_scale"],
                       "write_scale": row["write_scale"], "fetch_bytes_per_launch": row["fetch_bytes_per_launch"],
                       "write_bytes_per_launch": row["write_bytes_per_launch"],
                       "hbm_bytes_per_launch": row["hbm_bytes_per_launch"]}, f, indent=1)
        log(f"{w.name}: MFMA busy {row['mfma_busy_pct']:.1f} %, LDS conflicts {row['lds_bank_conflict_pct']:.2f} %, "
            f"HBM-side {row['hbm_bytes_per_launch'] / 1e6:.1f} MB (compulsory {comp / 1e6:.1f} MB)")

    L = [f"Calibration (256 MiB copy): FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}. "
         f"Kernel source hash {src_hash}.", "",
         "| workload | config | MFMA busy % | LDS bank-conflict % | HBM-side MB / launch (read + write) | "
         "compulsory MB | ratio | GB/s at hot time |",
         "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        gbps = f"{r['hbm_gbps_at_hot_time']:.0f}" if "hbm_gbps_at_hot_time" in r else "-"
        L.append(f"| {r['workload']} | {r['config']} | {r['mfma_busy_pct']:.1f} | {r['lds_bank_conflict_pct']:.2f} | "
                 f"{r['hbm_bytes_per_launch'] / 1e6:.1f} ({r['fetch_bytes_per_launch'] / 1e6:.1f} + "
                 f"{r['write_bytes_per_launch'] / 1e6:.1f}) | {r['compulsory_bytes'] / 1e6:.1f} | "
                 f"{r['hbm_bytes_per_launch'] / r['compulsory_bytes']:.2f} | {gbps} |")
    md = "\n".join(L) + "\n"
    print(md)
    with open(os.path.join(out, "counters.json"), "w") as f:
        json.dump({"fetch_scale": f_scale, "write_scale": w_scale, "rows": rows}, f, indent=1)
    if args.md:
        with open(args.md, "w") as f:
            f.write(md)
    return 0


if __name__ == "__main__":
    sys.exit(main())
