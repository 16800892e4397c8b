"""Timing protocol for every measured workload (one MI355X), beyond bench.py's one line.

For each workload, with the config gemm_f16 picks:
  * warm: 10 untimed calls and >= 50 ms of calls, then 7 trials of R back-to-back calls (R chosen so a trial
    lasts >= 20 ms), each trial bracketed by HIP events on the launch stream; the median
    trial gives us per call, TFLOP/s = 2MNK / t, and % of the dense fp16 MFMA peak
    (256 CU x 4096 FLOP/clk x 2.4 GHz = 2516.6 TFLOP/s) and of the measured MFMA ceiling;
  * cold: the same with >= 4 distinct (A, B, C) buffer sets totalling more than 288 MiB
    (more than the 256 MiB Infinity Cache), rotated call by call, so every call starts
    with its operands out of every cache;
  * phases: one more trial through the instrumented build (libtgemm_stamps.so); the
    stamps of its last call give, per workgroup, prologue / main loop / epilogue wall
    time, the shader clock the workgroup ran at, and the main loop's average per XCD;
  * split-K: where gemm_f16_ws would split (small output grids), the same timing through
    gemm_f16_ws with its planned config and split count;
  * context: torch.matmul (hipBLASLt) (+ relu_ when the workload has ReLU) timed the
    same way. Context only; never a target.
The MFMA ceiling is the library's MFMA probe (no memory traffic, N(0,1) binary16
operands) timed the same way, with its own clock from the stamps; its variants (synthetic
operands, 32x32x16 MFMAs, the GEMM's LDS read rate added) are reported beside it.

--ramp NAME instead records one event pair per call over a long back-to-back run of one
workload (twice, 2 s idle in between) and prints the mean per-call time in windows of
the run: from idle the GPU raises its clocks over the first tens of milliseconds of
load, so a timing that starts that early reads low. This sets how much warm-up the
other timings and bench.py need.

  python -m tiled_dense_gemm_04_amd.measure [--workloads a,b] [--no-cold] [--no-torch]
      [--json out.json] [--md out.md]
  python -m tiled_dense_gemm_04_amd.measure --ramp relu_4096 [--ramp-launches 3000]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
FP8_PEAK_TFLOPS = 256 * 8192 * 2.4e9 / 1e12   # dense fp8 MFMA peak (AMD: ~5.0 PFLOP/s)
HBM_PEAK_GBS = 8000.0
REALTIME_HZ = 100e6          # s_memrealtime
CACHE_BYTES = 288 << 20      # cold sets must exceed this in total (Infinity Cache: 256 MiB)
NUM_XCD = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_trials(torch, stream, call, trials=7, min_ms=20.0, warm=10, warm_ms=50.0):
    """Median microseconds per call over `trials` trials of R calls each, after at least
    `warm` calls and `warm_ms` of back-to-back calls (past the clock ramp from idle)."""
    for _ in range(warm):
        call(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            call(0)
        torch.cuda.synchronize()
    e0.record(stream)
    for i in range(5):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    est_ms = e0.elapsed_time(e1) / 5
    reps = max(5, math.ceil(min_ms / max(est_ms, 1e-3)))
    per = []
    for _ in range(trials):
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps * 1e3)
    return {"median_us": statistics.median(per), "min_us": min(per), "max_us": max(per),
            "calls_per_trial": reps, "trials": trials}


def graph_trials(torch, call, calls=64, trials=7, min_ms=20.0, warm_ms=50.0):
    """Median microseconds per call from replays of one HIP graph holding `calls` captured
    calls (issued on the current stream): GPU time without the host's per-call launch
    overhead, for kernels shorter than that overhead. `call(i)` must launch on the current
    stream."""
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call(i)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    t_end = time.perf_counter() + warm_ms * 1e-3
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    reps = max(1, math.ceil(min_ms / max(e0.elapsed_time(e1), 1e-3)))
    per = []
    for _ in range(trials):
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / (reps * calls) * 1e3)
    del g
    return {"median_us": statistics.median(per), "min_us": min(per), "max_us": max(per),
            "calls_per_trial": reps * calls, "trials": trials, "graph": True}


def ramp(torch, tg, w, stream, launches=3000, runs=2, idle_s=2.0):
    """Per-call durations (us) of `runs` back-to-back runs of `launches` calls each."""
    A, B = w.inputs()
    SA, SB = w.stored(A, B)
    a = torch.from_numpy(SA).cuda()
    b = torch.from_numpy(SB).cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    out = []
    for r in range(runs):
        if r:
            time.sleep(idle_s)
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(launches):
            tg.gemm_f16_ex(a, b, c, w.trans_a, w.trans_b, relu=w.relu, stream=stream)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        out.append([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(launches)])
        log(f"ramp run {r}: {launches} calls of {w.name}")
    return out


def ramp_markdown(w, runs, host) -> str:
    n = len(runs[0])
    edges = [0, 1, 20, 40, 60, 80, 100, 150, 200, 400, 700, 1000, 1500, 2000, 3000, 5000, 10000]
    edges = [e for e in edges if e < n] + [n]
    L = [f"Device: {host['device']}; {host['library']}; torch {host['torch']}.", "",
         f"{w.name} ({w.M}x{w.N}x{w.K}), {n} back-to-back calls per run, one event pair per call "
         "(the events add a small gap between calls); mean / min us per call in each window, "
         "elapsed ms at the window's end.", "",
         "| calls | " + " | ".join(f"run {r} mean | run {r} min | run {r} ms" for r in range(len(runs))) + " |",
         "|---|" + "---|---|---|" * len(runs)]
    for lo, hi in zip(edges[:-1], edges[1:]):
        cells = []
        for d in runs:
            seg = d[lo:hi]
            cells += [f"{statistics.mean(seg):.2f}", f"{min(seg):.2f}", f"{sum(d[:hi]) / 1e3:.1f}"]
        L.append(f"| {lo}-{hi} | " + " | ".join(cells) + " |")
    return "\n".join(L) + "\n"


def phases(stamps):
    """Summary of a stamp table (rows = workgroups of one launch)."""
    import numpy as np
    st = stamps[stamps[:, 7] == 1].astype(np.float64)
    if len(st) == 0:
        return None
    t0 = st[:, 0].min()
    pro = (st[:, 1] - st[:, 0]) / REALTIME_HZ * 1e6
    loop = (st[:, 2] - st[:, 1]) / REALTIME_HZ * 1e6
    epi = (st[:, 3] - st[:, 2]) / REALTIME_HZ * 1e6
    clk = st[:, 4] / np.maximum(st[:, 2] - st[:, 0], 1) * REALTIME_HZ / 1e9
    ids = np.nonzero(stamps[:, 7] == 1)[0]
    per_xcd = [float(loop[ids % NUM_XCD == x].mean()) if np.any(ids % NUM_XCD == x) else None
               for x in range(NUM_XCD)]
    iters = float(st[:, 5].mean())
    return {
        "workgroups": int(len(st)),
        "prologue_us": float(pro.mean()),
        "loop_us": float(loop.mean()),
        "loop_us_max": float(loop.max()),
        "epilogue_us": float(epi.mean()),
        "span_us": float((st[:, 3].max() - t0) / REALTIME_HZ * 1e6),
        "start_spread_us": float((st[:, 0].max() - t0) / REALTIME_HZ * 1e6),
        "loop_iterations": iters,
        "ns_per_iteration": float(loop.mean() / max(iters, 1) * 1e3),
        "shader_clock_ghz": float(clk.mean()),
        "loop_us_per_xcd": per_xcd,
    }


PROBE_VARIANTS = [
    ("operands", "N(0,1) binary16 operands (the workloads' distribution), 16x16x32 MFMAs"),
    ("synthetic", "pseudo-random register operands (random sign and mantissa, magnitudes 2^-2 to 2^1), 16x16x32"),
    ("operands_32x32", "N(0,1) operands, 32x32x16 MFMAs (half as many, twice the FLOP each)"),
    ("lds_reads", "N(0,1) operands, 16x16x32, plus the 256 x 256 GEMM's LDS read rate (6 ds_read_b128 "
                  "per 16 MFMAs per wave)"),
]


def measure_probe(torch, tg, stream, mode="synthetic", operands=None, blocks=512, iters=2000):
    out = torch.empty(blocks * tg.PROBE_THREADS, dtype=torch.float32, device="cuda")
    flop = blocks * (tg.PROBE_THREADS // 64) * iters * tg.PROBE_MFMA_PER_ITER * tg.PROBE_FLOP_PER_MFMA

    def call(_i, library=None):
        tg.tgemm_mfma_probe_ex(mode, blocks, iters, out, operands=operands, stream=stream, library=library)

    t = timed_trials(torch, stream, call)
    S = tg.stamps_lib()
    timed_trials(torch, stream, lambda i: call(i, S), trials=1, warm=2)
    ph = phases(tg.tgemm_stamps_read(blocks))
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        raise RuntimeError("MFMA probe produced non-finite values")
    tf = flop / (t["median_us"] * 1e-6) / 1e12
    res = {"mode": mode, "blocks": blocks, "iters": iters, "flop": flop, **t, "tflops": tf,
           "pct_of_peak": 100 * tf / PEAK_TFLOPS, "phases": ph}
    log(f"MFMA probe ({mode}): {t['median_us']:.1f} us/launch, {tf:.1f} TFLOP/s ({100 * tf / PEAK_TFLOPS:.1f} % of "
        f"{PEAK_TFLOPS:.1f}); shader clock {ph['shader_clock_ghz'] if ph else float('nan'):.3f} GHz")
    return res


def measure_probes(torch, tg, W, stream):
    """Every probe variant; the one on N(0,1) operands is the ceiling the GEMMs are held to
    (same data distribution as the workloads, no memory traffic)."""
    A, _ = W.make_inputs(tg.PROBE_THREADS, 1, 64, "normal", 1.0, seed=40)
    ops = torch.from_numpy(A).cuda().contiguous()
    variants = [measure_probe(torch, tg, stream, mode, None if mode == "synthetic" else ops)
                for mode, _ in PROBE_VARIANTS]
    return {"ceiling": variants[0], "variants": variants}


def measure_workload(torch, tg, W, w, stream, cold=True, with_torch=True, ceiling=None):
    SA, SB = w.stored(*w.inputs())
    a = torch.from_numpy(SA).cuda()
    b = torch.from_numpy(SB).cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    cfg = tg.tgemm_select_config_ex(w.trans_a, w.trans_b, w.M, w.N, w.K, a.data_ptr(), a.stride(0),
                                    b.data_ptr(), b.stride(0), c.data_ptr(), c.stride(0))
    desc = tg.tgemm_config_desc(cfg)
    res = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "relu": w.relu, "flop": w.flop,
           "trans_a": w.trans_a, "trans_b": w.trans_b,
           "config": desc["name"], "config_index": cfg,
           "compulsory_bytes": 2 * (w.M * w.K + w.K * w.N + w.M * w.N)}

    def tf(us):
        return w.flop / (us * 1e-6) / 1e12

    def gemm(x, y, z, library=None):
        tg.gemm_f16_ex(x, y, z, w.trans_a, w.trans_b, relu=w.relu, stream=stream, library=library)

    hot = timed_trials(torch, stream, lambda i: gemm(a, b, c))
    res["hot"] = {**hot, "tflops": tf(hot["median_us"]), "pct_of_peak": 100 * tf(hot["median_us"]) / PEAK_TFLOPS}
    if ceiling:
        res["hot"]["pct_of_mfma_ceiling"] = 100 * tf(hot["median_us"]) / ceiling
    log(f"{w.name}: {desc['name']} hot {hot['median_us']:.2f} us ({tf(hot['median_us']):.1f} TFLOP/s)")

    plan = tg.tgemm_split_plan(w.trans_a, w.trans_b, w.M, w.N, w.K, a.data_ptr(), a.stride(0), b.data_ptr(),
                               b.stride(0), c.data_ptr(), c.stride(0))
    if plan[1] > 1:
        ws = tg.workspace_for(plan[2], a.device, stream.cuda_stream)
        sk = timed_trials(torch, stream, lambda i: tg.gemm_f16_ws(a, b, c, w.trans_a, w.trans_b, relu=w.relu,
                                                                stream=stream, workspace=ws))
        res["split_k"] = {**sk, "config": tg.tgemm_config_desc(plan[0])["name"], "splits": plan[1],
                          "workspace_bytes": plan[2], "tflops": tf(sk["median_us"]),
                          "pct_of_peak": 100 * tf(sk["median_us"]) / PEAK_TFLOPS}
        log(f"{w.name}: split-K {plan[1]} x {res['split_k']['config']} {sk['median_us']:.2f} us")

    if cold:
        per_set = res["compulsory_bytes"]
        nsets = max(4, math.ceil(CACHE_BYTES / per_set) + 1)
        sets = [(a.clone(), b.clone(), torch.empty_like(c)) for _ in range(nsets)]
        cold_t = timed_trials(torch, stream, lambda i: gemm(*sets[i % nsets]))
        res["cold"] = {**cold_t, "sets": nsets, "bytes_total": nsets * per_set,
                       "tflops": tf(cold_t["median_us"]), "pct_of_peak": 100 * tf(cold_t["median_us"]) / PEAK_TFLOPS}
        log(f"{w.name}: cold ({nsets} sets, {nsets * per_set / 2**20:.0f} MiB) {cold_t['median_us']:.2f} us")
        del sets
        torch.cuda.empty_cache()

    S = tg.stamps_lib()
    timed_trials(torch, stream, lambda i: gemm(a, b, c, library=S), trials=1, warm=3)
    nwg = tg.tgemm_num_workgroups(cfg, w.M, w.N)
    res["phases"] = phases(tg.tgemm_stamps_read(nwg))
    if res["phases"]:
        ph = res["phases"]
        log(f"{w.name}: phases prologue {ph['prologue_us']:.2f} loop {ph['loop_us']:.2f} "
            f"epilogue {ph['epilogue_us']:.2f} us, clock {ph['shader_clock_ghz']:.3f} GHz")

    if with_torch:
        opa = a.t() if w.trans_a else a
        opb = b.t() if w.trans_b else b

        def tmm(_i):
            r = torch.matmul(opa, opb)
            if w.relu:
                torch.relu_(r)
        with torch.cuda.stream(stream):
            th = timed_trials(torch, stream, tmm)
        res["torch_matmul"] = {**th, "tflops": tf(th["median_us"]), "note": "context only (hipBLASLt"
                               + (" + separate relu_ kernel)" if w.relu else ")")}
        log(f"{w.name}: torch.matmul{'+relu_' if w.relu else ''} {th['median_us']:.2f} us")
    del a, b, c
    torch.cuda.empty_cache()
    return res


def measure_grouped(torch, tg, w, stream, with_torch=True):
    """One grouped workload: gemm_f16_grouped (one launch) against the same GEMMs issued
    one gemm_f16 call each, and (context) a loop of torch.matmul (+ relu_)."""
    ins = w.inputs()
    probs = [(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()) for A, B in ins]
    outs = [torch.empty((a.shape[0], b.shape[1]), dtype=torch.float16, device="cuda") for a, b in probs]
    trip = [(a, b, c) for (a, b), c in zip(probs, outs)]

    def tf(us):
        return w.flop / (us * 1e-6) / 1e12

    g = timed_trials(torch, stream, lambda i: tg.gemm_f16_grouped(trip, relu=w.relu, stream=stream))
    seq = timed_trials(torch, stream, lambda i: [tg.gemm_f16(a, b, c, relu=w.relu, stream=stream) for a, b, c in trip])
    res = {"workload": w.name, "Ms": list(w.Ms), "N": w.N, "K": w.K, "relu": w.relu, "flop": w.flop,
           "grouped": {**g, "tflops": tf(g["median_us"]), "pct_of_peak": 100 * tf(g["median_us"]) / PEAK_TFLOPS},
           "sequential": {**seq, "tflops": tf(seq["median_us"])}}
    log(f"{w.name}: grouped {g['median_us']:.2f} us, one call per GEMM {seq['median_us']:.2f} us")
    if with_torch:
        def tmm(_i):
            for a, b in probs:
                r = torch.matmul(a, b)
                if w.relu:
                    torch.relu_(r)
        with torch.cuda.stream(stream):
            th = timed_trials(torch, stream, tmm)
        res["torch_matmul"] = {**th, "tflops": tf(th["median_us"]), "note": "context only"}
    del probs, outs, trip
    torch.cuda.empty_cache()
    return res


def measure_fp8(torch, tg, w, stream, with_torch=True):
    """One fp8 workload. Block-scaled GEMM (w.linear False): the default config and every
    other fp8 config, hot. Linear step (w.linear True): the 1 x 128 quantizer alone
    (against HBM bandwidth), the GEMM on the quantized x, and quantizer + GEMM together.
    Context: torch._scaled_mm (hipBLASLt fp8, one scale per tensor) where it runs."""
    M, N, K = w.M, w.N, w.K
    KB = -(-K // 128)

    def tf(us):
        return w.flop / (us * 1e-6) / 1e12

    res = {"workload": w.name, "M": M, "N": N, "K": K, "relu": w.relu, "flop": w.flop, "linear": w.linear}
    if w.linear:
        x, Wc, SW = w.inputs()
        xd, wd, swd = torch.from_numpy(x).cuda(), torch.from_numpy(Wc).cuda(), torch.from_numpy(SW).cuda()
        xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sx = torch.empty((M, KB), dtype=torch.float32, device="cuda")
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        # The quantizer is shorter than the host's per-call overhead through the Python
        # binding, so back-to-back calls would time the host: time it from graph replays.
        q = graph_trials(torch, lambda i: tg.quant_fp8_block(xd, 1, xq, sx))
        q_host = timed_trials(torch, stream, lambda i: tg.quant_fp8_block(xd, 1, xq, sx, stream=stream))
        qbytes = 2 * M * K + M * K + 4 * M * KB
        res["quant"] = {**q, "bytes": qbytes, "gbs": qbytes / (q["median_us"] * 1e-6) / 1e9,
                        "back_to_back_us": q_host["median_us"]}
        res["quant"]["pct_of_hbm"] = 100 * res["quant"]["gbs"] / HBM_PEAK_GBS
        a, sa, b, sb = xq, sx, wd, swd
        lin = timed_trials(torch, stream, lambda i: (tg.quant_fp8_block(xd, 1, xq, sx, stream=stream),
                                                     tg.gemm_fp8_block(xq, sx, wd, swd, c, relu=w.relu,
                                                                       stream=stream)))
        res["linear_total"] = {**lin, "tflops": tf(lin["median_us"])}
        log(f"{w.name}: quant {q['median_us']:.2f} us ({res['quant']['gbs']:.0f} GB/s), "
            f"quant + gemm {lin['median_us']:.2f} us")
    else:
        A, SA, B, SB = w.inputs()
        a, sa = torch.from_numpy(A).cuda(), torch.from_numpy(SA).cuda()
        b, sb = torch.from_numpy(B).cuda(), torch.from_numpy(SB).cuda()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
    cfg = tg.tgemm_fp8_select_config(M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0), c.data_ptr(),
                                     c.stride(0))
    res["config"] = tg.tgemm_fp8_config_desc(cfg)["name"] if cfg >= 0 else "generic"
    h = timed_trials(torch, stream, lambda i: tg.gemm_fp8_block(a, sa, b, sb, c, relu=w.relu, stream=stream))
    res["hot"] = {**h, "tflops": tf(h["median_us"]), "pct_of_peak": 100 * tf(h["median_us"]) / FP8_PEAK_TFLOPS}
    log(f"{w.name}: gemm_fp8_block {h['median_us']:.2f} us ({res['hot']['tflops']:.1f} TFLOP/s) [{res['config']}]")
    if cfg >= 0:
        S = tg.stamps_lib()
        timed_trials(torch, stream, lambda i: tg.gemm_fp8_block(a, sa, b, sb, c, relu=w.relu, stream=stream,
                                                                library=S), trials=1, warm=3)
        d = tg.tgemm_fp8_config_desc(cfg)
        res["phases"] = phases(tg.tgemm_stamps_read(-(-M // d["block_m"]) * -(-N // d["block_n"])))
        if res["phases"]:
            ph = res["phases"]
            log(f"{w.name}: phases prologue {ph['prologue_us']:.2f} loop {ph['loop_us']:.2f} "
                f"epilogue {ph['epilogue_us']:.2f} us, clock {ph['shader_clock_ghz']:.3f} GHz, "
                f"{ph['ns_per_iteration']:.0f} ns per k-tile")
    res["per_config"] = {}
    for idx in range(tg.tgemm_fp8_num_configs()):
        if idx == cfg:
            continue
        # configs left out of the product library run from the tooling build (marked "(t)")
        d = tg.tgemm_fp8_config_desc(idx)
        lib = None if d["built"] else tg.stamps_lib()
        t = timed_trials(torch, stream, lambda i, idx=idx, lib=lib: tg.gemm_fp8_block(
            a, sa, b, sb, c, relu=w.relu, stream=stream, cfg=idx, library=lib), trials=5)
        res["per_config"][d["name"] + ("" if d["built"] else " (t)")] = t["median_us"]
    if with_torch and not w.linear:
        try:
            f8 = torch.float8_e4m3fn
            a8, bt8 = a.view(f8), b.view(f8).t()
            one = torch.ones((), dtype=torch.float32, device="cuda")
            with torch.cuda.stream(stream):
                th = timed_trials(torch, stream, lambda i: torch._scaled_mm(a8, bt8, one, one, out_dtype=torch.float16))
            res["torch_scaled_mm"] = {**th, "tflops": tf(th["median_us"]), "note": "context only; one scale per tensor"}
        except Exception as e:  # not every torch build runs fp8 GEMMs on this device
            res["torch_scaled_mm"] = {"error": f"{type(e).__name__}: {e}"[:160]}
    torch.cuda.empty_cache()
    return res


def fp8_markdown(fp8) -> str:
    L = ["", f"fp8 (E4M3) block-scaled path (gemm_fp8_block; peak = dense fp8 MFMA {FP8_PEAK_TFLOPS:.1f} TFLOP/s):",
         "", "| workload | config | hot us (min-max) | TFLOP/s | % fp8 peak | other configs us | "
         "quant_fp8_block us from graph replays (GB/s, % of 8 TB/s; back-to-back calls) | quant + GEMM us | "
         "torch._scaled_mm us (context) |",
         "|---|---|---|---|---|---|---|---|---|"]
    for r in fp8:
        h = r["hot"]
        others = ", ".join(f"{k} {v:.2f}" for k, v in r.get("per_config", {}).items()) or "-"
        q = r.get("quant")
        qs = (f"{q['median_us']:.2f} ({q['gbs']:.0f}, {q['pct_of_hbm']:.1f} %; {q['back_to_back_us']:.2f})"
              if q else "-")
        lt = f"{r['linear_total']['median_us']:.2f}" if "linear_total" in r else "-"
        ts = r.get("torch_scaled_mm")
        tss = "-" if not ts else (f"{ts['median_us']:.2f}" if "median_us" in ts else ts["error"])
        L.append(f"| {r['workload']} ({r['M']}x{r['N']}x{r['K']}) | {r['config']} | {h['median_us']:.2f} "
                 f"({h['min_us']:.2f}-{h['max_us']:.2f}) | {h['tflops']:.1f} | {h['pct_of_peak']:.1f} | {others} | "
                 f"{qs} | {lt} | {tss} |")
    L += ["", "Phases of gemm_fp8_block (instrumented build, means over workgroups):", "",
          "| workload | workgroups | prologue us | main loop us (max) | epilogue us | launch span us | "
          "ns per k-tile (128 k) | shader clock GHz |", "|---|---|---|---|---|---|---|---|"]
    for r in fp8:
        ph = r.get("phases")
        if ph:
            L.append(f"| {r['workload']} | {ph['workgroups']} | {ph['prologue_us']:.2f} | {ph['loop_us']:.2f} "
                     f"({ph['loop_us_max']:.2f}) | {ph['epilogue_us']:.2f} | {ph['span_us']:.2f} | "
                     f"{ph['ns_per_iteration']:.0f} | {ph['shader_clock_ghz']:.3f} |")
    return "\n".join(L) + "\n"


def markdown(results, probe, host, grouped=None) -> str:
    L = []
    L.append(f"Device: {host['device']}; {host['library']}; torch {host['torch']}.")
    L.append("")
    if probe:
        c = probe["ceiling"]
        ph = c.get("phases") or {}
        L.append(f"MFMA ceiling (probe: {c['blocks']} workgroups x 8 waves, {c['iters']} rounds of 16 "
                 f"independent 16x16x32 fp16 MFMAs, N(0,1) binary16 operands, no memory traffic): "
                 f"**{c['tflops']:.1f} TFLOP/s** = {c['pct_of_peak']:.1f} % of {PEAK_TFLOPS:.1f}, "
                 f"shader clock {ph.get('shader_clock_ghz', float('nan')):.3f} GHz (s_memtime / s_memrealtime).")
        L.append("")
        L.append("Probe variants (same FLOP per launch; `tgemm_mfma_probe_ex` of the tooling build):")
        L.append("")
        L.append("| variant | TFLOP/s | % of peak | shader clock GHz |")
        L.append("|---|---|---|---|")
        desc = dict(PROBE_VARIANTS)
        for v in probe["variants"]:
            vph = v.get("phases") or {}
            L.append(f"| {desc[v['mode']]} | {v['tflops']:.1f} | {v['pct_of_peak']:.1f} | "
                     f"{vph.get('shader_clock_ghz', float('nan')):.3f} |")
        L.append("")
    L.append("| workload | config | hot us (min-max) | TFLOP/s | % peak | % MFMA ceiling | cold us | "
             "split-K (gemm_f16_ws) us | hipBLASLt us (context) |")
    L.append("|---|---|---|---|---|---|---|---|---|")
    for r in results:
        h = r["hot"]
        cold = f"{r['cold']['median_us']:.2f} ({r['cold']['sets']} sets)" if "cold" in r else "-"
        th = f"{r['torch_matmul']['median_us']:.2f}" if "torch_matmul" in r else "-"
        ceil = f"{h['pct_of_mfma_ceiling']:.1f}" if "pct_of_mfma_ceiling" in h else "-"
        sk = r.get("split_k")
        sks = (f"{sk['median_us']:.2f} ({sk['splits']} x {sk['config']}, {sk['tflops']:.1f} TFLOP/s)"
               if sk else "- (no split)")
        L.append(f"| {r['workload']} ({r['M']}x{r['N']}x{r['K']}) | {r['config']} | {h['median_us']:.2f} "
                 f"({h['min_us']:.2f}-{h['max_us']:.2f}) | {h['tflops']:.1f} | {h['pct_of_peak']:.1f} | {ceil} | "
                 f"{cold} | {sks} | {th} |")
    if grouped:
        L.append("")
        L.append("Grouped GEMMs (gemm_f16_grouped, one launch) against one gemm_f16 call per GEMM:")
        L.append("")
        L.append("| workload | rows per GEMM | grouped us | TFLOP/s | % peak | one call each us | "
                 "hipBLASLt loop us (context) |")
        L.append("|---|---|---|---|---|---|---|")
        for r in grouped:
            th = f"{r['torch_matmul']['median_us']:.2f}" if "torch_matmul" in r else "-"
            L.append(f"| {r['workload']} (N {r['N']}, K {r['K']}) | {' '.join(str(m) for m in r['Ms'])} | "
                     f"{r['grouped']['median_us']:.2f} | {r['grouped']['tflops']:.1f} | "
                     f"{r['grouped']['pct_of_peak']:.1f} | {r['sequential']['median_us']:.2f} | {th} |")
    L.append("")
    L.append("Phases of the last call of one more trial, instrumented build (means over workgroups):")
    L.append("")
    L.append("| workload | workgroups | prologue us | main loop us (max) | epilogue us | launch span us | "
             "ns per k-tile | shader clock GHz | main loop us per XCD 0..7 |")
    L.append("|---|---|---|---|---|---|---|---|---|")
    for r in results:
        ph = r.get("phases")
        if not ph:
            continue
        xcd = " ".join(f"{v:.1f}" if v is not None else "-" for v in ph["loop_us_per_xcd"])
        L.append(f"| {r['workload']} | {ph['workgroups']} | {ph['prologue_us']:.2f} | {ph['loop_us']:.2f} "
                 f"({ph['loop_us_max']:.2f}) | {ph['epilogue_us']:.2f} | {ph['span_us']:.2f} | "
                 f"{ph['ns_per_iteration']:.0f} | {ph['shader_clock_ghz']:.3f} | {xcd} |")
    return "\n".join(L) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", default=None, help="comma-separated names (default: all)")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-torch", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--json", default=None)
    ap.add_argument("--md", default=None)
    ap.add_argument("--ramp", default=None, metavar="WORKLOAD", help="only the clock-ramp trace of WORKLOAD")
    ap.add_argument("--ramp-launches", type=int, default=3000)
    args = ap.parse_args()

    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg

    if not torch.cuda.is_available():
        log("measure needs a GPU")
        return 1
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    works = W.all_workloads()
    if args.workloads:
        keep = set(args.workloads.split(","))
        works = [w for w in works if w.name in keep]
    host = {"device": torch.cuda.get_device_name(0), "library": tg.tgemm_version(), "torch": torch.__version__,
            "time": time.strftime("%Y-%m-%d %H:%M:%S")}
    if args.ramp:
        w = W.by_name(args.ramp)
        md = ramp_markdown(w, ramp(torch, tg, w, stream, args.ramp_launches), host)
        print(md)
        if args.md:
            with open(args.md, "w") as f:
                f.write(md)
        return 0
    probe = None if args.no_probe else measure_probes(torch, tg, W, stream)
    ceiling = probe["ceiling"]["tflops"] if probe else None
    results = [measure_workload(torch, tg, W, w, stream, cold=not args.no_cold, with_torch=not args.no_torch,
                                ceiling=ceiling) for w in works]
    grouped = [measure_grouped(torch, tg, gw, stream, with_torch=not args.no_torch)
               for gw in W.GROUPED_WORKLOADS.values()
               if not args.workloads or gw.name in set(args.workloads.split(","))]
    fp8 = [measure_fp8(torch, tg, fw, stream, with_torch=not args.no_torch)
           for fw in W.FP8_WORKLOADS.values()
           if not args.workloads or fw.name in set(args.workloads.split(","))]
    md = markdown(results, probe, host, grouped) + (fp8_markdown(fp8) if fp8 else "")
    print(md)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"host": host, "probe": probe, "results": results, "grouped": grouped, "fp8": fp8}, f,
                      indent=1)
    if args.md:
        with open(args.md, "w") as f:
            f.write(md)
    return 0


if __name__ == "__main__":
    sys.exit(main())
