#!/usr/bin/env python3
"""Benchmark: fp16 GEMM + fused ReLU through libtgemm on one MI355X.

One step = one gemm_f16 call over the whole workload (C = ReLU(A @ B), M = N = K = 4096,
fp16 inputs drawn N(0,1) from seed 2, fp32 accumulate, fp16 out, row-major), inputs
already resident in HBM. W untimed warm-up steps, then exactly K timed steps bracketed
by device synchronisation. Prints ONE JSON line on stdout; details go to stderr.

From idle, the board's power control brings the clocks to their sustained level over the
first few hundred calls (at 4096^3, calls 20-200 run 10-30 % slower than the steady state).
Before the W counted warm-up steps, a settle phase therefore runs back-to-back calls for
--settle-ms of wall time (default 300 ms), untimed, so that even a short run (W = 5) times
the sustained state; the JSON line reports it as "settle" and names the clock state.

  value            = 2*M*N*K*steps / wall time of the timed steps, in TFLOP/s
  roofline.achieved = 2*M*N*K / mean kernel duration, from HIP events recorded on the
                     stream the kernels are launched on, against the dense fp16 MFMA peak
  cpu_baseline     = the CPU oracle (as it stands) timed on the host on a slab of rows of
                     the same workload, in TFLOP/s: "cores" = the threads it used; also
                     the host's CPU count and model, and the oracle on one thread over the
                     1024^3 GEMM + ReLU (the pages' first example) for a per-core figure

--workload also takes the fp8 block-scaled workloads (fp8_block_4096, fp8_block_relu_8192:
one gemm_fp8_block call per step on pre-quantized E4M3 inputs; fp8_linear_4096: the 1 x 128
quantizer plus the GEMM per step); their line is priced against the dense fp8 MFMA peak
(256 CUs x 8192 FLOP/clk/CU x 2.4 GHz = 5033.2 TFLOP/s). The default stays the fp16 4096^3
GEMM + ReLU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM+ReLU TFLOP/s at 4096^3 on 1 MI355X; % of dense fp16 MFMA peak"
# Dense fp16 MFMA peak of MI355X: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz (AMD's ~2.5 PFLOP/s).
PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
FP8_PEAK_TFLOPS = 256 * 8192 * 2.4e9 / 1e12
PROFILES = os.path.join(ROOT, "profiles")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the device code and the config lists (not the host-side selector), so
    profiles taken on a kernel stay valid while only the host logic changes."""
    h = hashlib.sha256()
    for f in ("tgemm_kernels.hip", "tgemm_device.h", "tgemm_fp8.hip", "tgemm_internal.h", "tgemm_configs.h"):
        with open(os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, cfg_name: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"traffic_{cfg_name}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        eprint(f"traffic counters in {path} are from another kernel version; reporting null")
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """The host the oracle runs on: logical CPUs, the ones this process may use, the model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"host_cpus": os.cpu_count(), "host_cpus_usable": usable, "cpu_model": model}


def one_thread_1024():
    """The oracle on one thread over relu_1024 (1024^3 GEMM + ReLU, N(0,1), seed 1): TFLOP/s."""
    import oracle
    import tgemm_workloads as W

    w = W.by_name("relu_1024")
    A, B = w.inputs()
    t = time.perf_counter()
    oracle.default().gemm(A, B, w.relu, nthreads=1)
    dt = time.perf_counter() - t
    eprint(f"cpu oracle, one thread, relu_1024: {dt:.2f} s ({w.flop / dt / 1e9:.2f} GFLOP/s)")
    return {"workload": "relu_1024", "threads": 1, "seconds": round(dt, 3), "value": w.flop / dt / 1e12,
            "unit": "TFLOP/s"}


def cpu_baseline(A, B, relu, c_gpu_bits, target_s: float):
    """Time the oracle on the first R rows of the workload; R sized for ~target_s."""
    import numpy as np
    import oracle

    orc = oracle.default()
    threads = orc.max_threads()
    M, K = A.shape
    N = B.shape[1]
    # calibrate on two slab sizes so the one-off decode of B cancels out of the rate
    times = {}
    for r in (16, 64):
        t = time.perf_counter()
        orc.gemm(A[:r], B, relu)
        times[r] = time.perf_counter() - t
    rate = 2.0 * (64 - 16) * N * K / max(times[64] - times[16], 1e-9)
    rows = int(min(M, max(64, rate * target_s / (2.0 * N * K))))
    t = time.perf_counter()
    ref = orc.gemm(A[:rows], B, relu)
    dt = time.perf_counter() - t
    flops = 2.0 * rows * N * K
    rep = oracle.compare(c_gpu_bits[:rows], ref, K)
    eprint(f"cpu oracle: {rows} rows x {N} x {K} in {dt:.2f} s on {threads} threads "
           f"({flops / dt / 1e9:.2f} GFLOP/s); GPU rows vs oracle: {rep}")
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {M} rows of the same workload (all N={N} columns, K={K}), "
                  f"{dt:.1f} s; GPU output on those rows vs oracle: {rep['fails']} tolerance failures",
        **host_cpu(),
        "per_core": one_thread_1024(),
    }


def cpu_baseline_fp8(A, SA, B, SB, relu, c_gpu_bits, target_s: float):
    """The fp8 oracle on the first R rows (codes as given), R sized for ~target_s."""
    import oracle

    orc = oracle.default()
    threads = orc.max_threads()
    M, K = A.shape
    N = B.shape[0]
    t = time.perf_counter()
    orc.gemm_fp8(A[:8], SA[:8], B, SB, relu)
    rate = 2.0 * 8 * N * K / max(time.perf_counter() - t, 1e-9)
    rows = int(min(M, max(8, rate * target_s / (2.0 * N * K))))
    t = time.perf_counter()
    ref = orc.gemm_fp8(A[:rows], SA[:rows], B, SB, relu)
    dt = time.perf_counter() - t
    flops = 2.0 * rows * N * K
    rep = oracle.compare_fp8(c_gpu_bits[:rows], ref, orc.fp8_bound(A[:rows], SA[:rows], B, SB))
    eprint(f"cpu fp8 oracle: {rows} rows x {N} x {K} in {dt:.2f} s on {threads} threads "
           f"({flops / dt / 1e9:.2f} GFLOP/s); GPU rows vs oracle: {rep}")
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {M} rows of the same workload (all N={N} columns, K={K}), "
                  f"{dt:.1f} s; GPU output on those rows vs oracle: {rep['fails']} tolerance failures",
        **host_cpu(),
    }


def settle(step, torch, ms: float) -> dict:
    """Untimed back-to-back calls for >= ms of wall time, so the clocks reach their
    sustained level before the counted warm-up."""
    torch.cuda.synchronize()
    calls, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            step()
        calls += 16
        torch.cuda.synchronize()
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "calls": calls}


def clock_state(st: dict, warmup: int) -> str:
    return (f"settled: {st['calls']} untimed back-to-back calls ({st['ms']} ms) before the {warmup} counted "
            f"warm-up steps, so the timed steps run at the sustained clock")


def bench_fp8(args, W, tg, torch, np) -> int:
    w = W.FP8_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    if w.linear:
        x, Bc, SB = w.inputs()
        xd = torch.from_numpy(x).to(dev)
        a = torch.empty((w.M, w.K), dtype=torch.uint8, device=dev)
        sa = torch.empty((w.M, -(-w.K // 128)), dtype=torch.float32, device=dev)
        A = SA = None
    else:
        A, SA, Bc, SB = w.inputs()
        a, sa = torch.from_numpy(A).to(dev), torch.from_numpy(SA).to(dev)
    b, sb = torch.from_numpy(Bc).to(dev), torch.from_numpy(SB).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    cfg = tg.tgemm_fp8_select_config(w.M, w.N, w.K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0),
                                     c.data_ptr(), c.stride(0))
    cfg_name = tg.tgemm_fp8_config_desc(cfg)["name"] if cfg >= 0 else "generic"
    eprint(f"{torch.cuda.get_device_name(dev)}; {tg.tgemm_version()}; fp8 workload {w.name} "
           f"{w.M}x{w.N}x{w.K} relu={w.relu} linear={w.linear}; config {cfg_name}")

    def step():
        if w.linear:
            tg.quant_fp8_block(xd, 1, a, sa, stream=stream)
        tg.gemm_fp8_block(a, sa, b, sb, c, relu=w.relu, stream=stream)

    st = settle(step, torch, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps
    value = w.flop * args.steps / wall / 1e12
    achieved = w.flop / (step_ms * 1e-3) / 1e12
    eprint(f"wall {wall * 1e3:.2f} ms for {args.steps} steps -> {value:.1f} TFLOP/s; event mean "
           f"{step_ms * 1e3:.2f} us/step -> {achieved:.1f} TFLOP/s ({100 * achieved / FP8_PEAK_TFLOPS:.1f} % of "
           f"{FP8_PEAK_TFLOPS:.1f})")
    out = {
        "metric": f"fp8 E4M3 block-scaled GEMM TFLOP/s at {w.M}x{w.N}x{w.K} on 1 MI355X; % of dense fp8 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "relu": w.relu, "linear": w.linear,
                   "inputs": (f"x fp16 N(0,1), weight E4M3 codes + 128x128 scales, seed {w.seed}" if w.linear else
                              f"E4M3 codes + 1x128 / 128x128 float32 scales, seed {w.seed}"),
                   "accumulate": "fp32 per 128-wide scale block", "kernel_config": cfg_name,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * achieved / FP8_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(FP8_PEAK_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(w.name, cfg_name), "kernel_us": round(step_ms * 1e3, 3),
                     "kernel_source_hash": kernel_source_hash()},
        "settle": st,
        "clock_state": clock_state(st, args.warmup),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and not w.linear:
        out["cpu_baseline"] = cpu_baseline_fp8(A, SA, Bc, SB, w.relu, c.cpu().numpy().view(np.uint16),
                                               args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="relu_4096",
                    help="relu_4096 (headline) or another name from tgemm_workloads.all_workloads()")
    ap.add_argument("--cfg", type=int, default=None, help="force a config index (sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed back-to-back calls for this long before the counted warm-up")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        n = args.copy_probe // 2
        src = torch.ones(n, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"copied {2 * n} bytes 5 times")
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "libtgemm runs on one GPU; there is no multi-GPU path (a GEMM split "
                                   "by output rows needs no communication: one process per GPU, each "
                                   "calling gemm_f16 on its own rows)",
                          "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        return 1
    if args.workload in W.FP8_WORKLOADS:
        return bench_fp8(args, W, tg, torch, np)
    w = W.by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A, B = w.inputs()
    SA, SB = w.stored(A, B)
    a = torch.from_numpy(SA).to(dev)
    b = torch.from_numpy(SB).to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(dev)
    cfg = args.cfg if args.cfg is not None else tg.tgemm_select_config_ex(
        w.trans_a, w.trans_b, w.M, w.N, w.K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0),
        c.data_ptr(), c.stride(0))
    cfg_name = tg.tgemm_config_desc(cfg)["name"]
    eprint(f"{torch.cuda.get_device_name(dev)}; {tg.tgemm_version()}; workload {w.name} "
           f"{w.M}x{w.N}x{w.K} relu={w.relu}; config {cfg} {cfg_name}")

    def step():
        tg.gemm_f16_ex(a, b, c, w.trans_a, w.trans_b, relu=w.relu, stream=stream, cfg=args.cfg)

    st = settle(step, torch, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    wall = t1 - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps
    flop = float(w.flop)
    value = flop * args.steps / wall / 1e12
    achieved = flop / (kern_ms * 1e-3) / 1e12
    eprint(f"wall {wall * 1e3:.2f} ms for {args.steps} steps -> {value:.1f} TFLOP/s; "
           f"event mean {kern_ms * 1e3:.2f} us/launch -> {achieved:.1f} TFLOP/s "
           f"({100 * achieved / PEAK_TFLOPS:.1f} % of {PEAK_TFLOPS:.1f})")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "M": w.M, "N": w.N, "K": w.K,
            "relu": w.relu,
            "trans_a": w.trans_a,
            "trans_b": w.trans_b,
            "inputs": f"fp16 iid {'N(0,%g)' % w.std if w.dist == 'normal' else 'U(-1,1)'} seed {w.seed}",
            "accumulate": "fp32",
            "kernel_config": cfg_name,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * achieved / PEAK_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": load_traffic(w.name, cfg_name),
            "kernel_us": round(kern_ms * 1e3, 3),
            "kernel_source_hash": kernel_source_hash(),
        },
        "settle": st,
        "clock_state": clock_state(st, args.warmup),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        c_bits = c.cpu().numpy().view(np.uint16)
        out["cpu_baseline"] = cpu_baseline(A, B, w.relu, c_bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
