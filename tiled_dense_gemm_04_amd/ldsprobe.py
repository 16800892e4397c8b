"""LDS bank-conflict probe: measures, on the GPU, the bank-conflict cycles of every LDS
access pattern in ldspatterns.py (calibration patterns and the kernels' own fragment,
staging and scale accesses) with the tooling build's tgemm_lds_probe, one dispatch per
distinct pattern, under rocprofv3 counters. Needs a GPU and rocprofv3.

  python -m tiled_dense_gemm_04_amd.ldsprobe --profile OUT_DIR [--json lds_bank_probe.json]

runs itself (`--run`) under `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE
SQ_INSTS_LDS` and writes, per distinct pattern (named by its first occurrence), the
conflict cycles and the LDS-busy cycles per instruction (counter / SQ_INSTS_LDS, so the
counters' sampling of units cancels). ldspatterns.bank_cycles is the model of these
numbers; tests/test_lds_bank_model.py holds it to the committed file.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COUNTERS = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS"]
ITERS, BLOCKS = 200, 256


def distinct(patterns):
    """Patterns keyed by (op, addresses, masks): the first name stands for all copies."""
    seen, out = {}, []
    for p in patterns:
        key = (p["op"], p["addrs"].tobytes(), tuple(p["active"]))
        if key not in seen:
            seen[key] = p["name"]
            out.append(p)
    return out, seen


def key_of(p):
    return (p["op"], p["addrs"].tobytes(), tuple(p["active"]))


def run():
    import torch

    import tiled_dense_gemm_04_amd as tg
    from tiled_dense_gemm_04_amd import ldspatterns as LP

    pats, _ = distinct(LP.all_patterns())
    out = torch.empty(BLOCKS, dtype=torch.float32, device="cuda")
    for i, p in enumerate(pats):
        tg.tgemm_lds_probe(p["op"], p["addrs"], p["active"], iters=ITERS, blocks=BLOCKS, out=out)
        if i % 200 == 0:
            torch.cuda.synchronize()
            print(f"{i} of {len(pats)} patterns", flush=True)
    torch.cuda.synchronize()
    print(f"done: {len(pats)} patterns", flush=True)


def per_dispatch(run_dir, name_filter="lds_probe"):
    """{dispatch id: {counter: value}} for the probe's dispatches."""
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_filter not in r["Kernel_Name"]:
                    continue
                d = vals.setdefault(int(r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return vals


def profile(out_dir, json_path):
    from tiled_dense_gemm_04_amd import ldspatterns as LP

    out_dir = os.path.abspath(out_dir)
    os.makedirs(out_dir, exist_ok=True)
    cmd = ["timeout", "-s", "KILL", "300", "rocprofv3", "--pmc", *COUNTERS, "--output-format", "csv", "-d", out_dir,
           "-o", "p", "--", sys.executable, "-m", "tiled_dense_gemm_04_amd.ldsprobe", "--run"]
    print(" ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run(cmd, cwd="/tmp", env=env)
    vals = per_dispatch(out_dir)
    if r.returncode != 0 and not (r.returncode in (139, -11) and vals):
        raise RuntimeError(f"rocprofv3 failed with status {r.returncode}")
    pats, _ = distinct(LP.all_patterns())
    ids = sorted(vals)
    if len(ids) != len(pats):
        raise RuntimeError(f"{len(ids)} probe dispatches for {len(pats)} patterns")
    res = {}
    for p, d in zip(pats, ids):
        v = vals[d]
        n = max(v.get("SQ_INSTS_LDS", 0.0), 1.0)
        res[p["name"]] = [round(v.get("SQ_LDS_BANK_CONFLICT", 0.0) / n, 3), round(v.get("SQ_LDS_IDX_ACTIVE", 0.0) / n, 3)]
    with open(json_path, "w") as f:
        f.write(json.dumps({"command": "python -m tiled_dense_gemm_04_amd.ldsprobe --profile OUT --json FILE",
                            "iters": ITERS, "blocks": BLOCKS, "counters": COUNTERS,
                            "columns": ["conflict cycles per instruction", "LDS-busy cycles per instruction"],
                            "patterns": res}, indent=None, separators=(",", ":")).replace('],"', '],\n"'))
    print(f"wrote {json_path}: {len(res)} patterns", flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--run", action="store_true", help="launch every distinct pattern once (profiled)")
    ap.add_argument("--profile", default=None, metavar="OUT_DIR")
    ap.add_argument("--json", default="lds_bank_probe.json")
    args = ap.parse_args()
    if args.run:
        run()
        return 0
    if args.profile:
        return profile(args.profile, args.json)
    ap.print_help()
    return 2


if __name__ == "__main__":
    sys.exit(main())
