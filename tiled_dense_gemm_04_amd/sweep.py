"""Offline config sweep: time every applicable table config of libtgemm on the measured
workloads and report the fastest per workload (the evidence behind the config choice in
tgemm_api.cpp's choose_fast). With --split, time split-K instead: the 256 x 256 and
128 x 128 ping-pong configs at 1, 2, 4 and 8 splits per output tile on small-grid shapes
(the evidence behind split_plan). Needs a GPU.

  python -m tiled_dense_gemm_04_amd.sweep [--out results.json] [--md out.md] [--torch] [--iters 30]
  python -m tiled_dense_gemm_04_amd.sweep --split [--md out.md]
  python -m tiled_dense_gemm_04_amd.sweep --choice [--md out.md]
  python -m tiled_dense_gemm_04_amd.sweep --write-table csrc/tgemm_choice.inc [--md out.md]
  python -m tiled_dense_gemm_04_amd.sweep --refit results.json --write-table tgemm_choice.inc

--choice checks the default config choice (fp16 choose_fast, fp8 fp8_choose) against the
candidate configs on shapes from 1024^2 to 6144^2, timed with the measurement protocol.

--write-table times every product config (those the product library compiles) on
TABLE_SHAPES and the measured workloads, fits the per-config cost model of the selector
(predicted microseconds a*R + b*R*k + c*O + d*k*O, R = ceil(tiles / 256), O = tiles / 256,
k = K / 1024; non-negative least squares on relative error), and writes the selector's
table (exact shapes with their fastest config, then the model coefficients) as C++ for
tgemm_api.cpp to include. The timings go to <table>.json beside it; --refit rewrites the
table from such a file without a GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12


def time_config(tg, torch, a, b, c, relu, cfg, iters, warmup=5, trans_a=False, trans_b=False):
    """Microseconds per launch of table config cfg: on the product library when it compiles
    the row, else on the tooling build (sweep-only variants)."""
    stream = torch.cuda.current_stream()
    library = None if tg.tgemm_config_desc(cfg)["built"] else tg.stamps_lib()

    def call():
        tg.gemm_f16_ex(a, b, c, trans_a, trans_b, relu=relu, cfg=cfg, library=library)

    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3  # us


CHOICE_SHAPES = [(1024, 1024, 4096), (1536, 1536, 4096), (2048, 2048, 4096), (2560, 2560, 4096),
                 (2048, 4096, 4096), (16384, 512, 4096), (3072, 3072, 4096), (3584, 3584, 2048),
                 (4096, 2560, 2048), (4095, 3000, 1000), (4096, 3072, 1024), (3072, 4096, 4096),
                 (5120, 4096, 4096), (6144, 6144, 4096)]
CHOICE_F16 = ["p64x128x64_s3_w2x2_p4_x1", "p64x128x32_s4_w2x2_p4_x1", "p128x128x64_s2_w2x2_p4_x1", "m128x128x32_s4_w2x4_p4_x1", "m256x128x32_s4_w2x4_p4_x1",
              "m128x256x32_s4_w2x4_p4_x1", "m256x192x32_s4_w2x4_p4_x1", "m256x256x32_s4_w2x4_p4_x1",
              "m256x256x32_s4_w2x4_p4_x0"]


def choice_sweep(md_path=None):
    """Time the candidate configs on CHOICE_SHAPES (fp16, then fp8 where the fast path
    applies) and report the default choice's loss against the fastest."""
    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg
    from tiled_dense_gemm_04_amd.measure import timed_trials

    stream = torch.cuda.current_stream()
    names = {c["name"]: i for i, c in enumerate(tg.configs())}
    L = ["# Default config choice against the candidates (one MI355X)", "",
         "Command (from the repository root): `python -m tiled_dense_gemm_04_amd.sweep --choice --md "
         "out/choice.md`", "",
         f"Device: {torch.cuda.get_device_name(0)}. Each config: 10 warm-up calls and >= 50 ms of calls, then 5",
         "trials of >= 20 ms (HIP events), median microseconds per call. * marks the config the library",
         "picks by itself; the last column is its loss against the fastest candidate.", "",
         "fp16 GEMM + ReLU (C = ReLU(A @ B), N(0,1) inputs):", "",
         "| M x N x K | " + " | ".join(CHOICE_F16) + " | loss |", "|---|" + "---|" * (len(CHOICE_F16) + 1)]
    for (M, N, K) in CHOICE_SHAPES:
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=5)
        a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        pick = tg.tgemm_config_desc(tg.tgemm_select_config(M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(),
                                                           b.stride(0), c.data_ptr(), c.stride(0)))["name"]
        t = {n: timed_trials(torch, stream, lambda i, n=n: tg.gemm_f16(a, b, c, cfg=names[n]), trials=5)["median_us"]
             for n in CHOICE_F16}
        best = min(t.values())
        loss = f"{100 * (t[pick] / best - 1):.1f} %" if pick in t else "-"
        L.append(f"| {M}x{N}x{K} | " + " | ".join(f"{v:.1f}{'*' if n == pick else ''}" for n, v in t.items())
                 + f" | {loss} |")
        print(L[-1], flush=True)
        del a, b, c
    nf8 = tg.tgemm_fp8_num_configs()
    f8names = [tg.tgemm_fp8_config_desc(i)["name"] for i in range(nf8)]
    L += ["", "fp8 block-scaled GEMM (E4M3 codes, 1 x 128 / 128 x 128 float32 scales):", "",
          "| M x N x K | " + " | ".join(f8names) + " | loss |", "|---|" + "---|" * (nf8 + 1)]
    for (M, N, K) in CHOICE_SHAPES:
        if N % 8 or K % 16:
            continue
        A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=5)
        a, sa, b, sb = (torch.from_numpy(x).cuda() for x in (A, SA, B, SB))
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        pick = tg.tgemm_fp8_select_config(M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0),
                                          c.data_ptr(), c.stride(0))
        t = [timed_trials(torch, stream, lambda i, k=k: tg.gemm_fp8_block(a, sa, b, sb, c, cfg=k), trials=5)["median_us"]
             for k in range(nf8)]
        L.append(f"| {M}x{N}x{K} | " + " | ".join(f"{v:.1f}{'*' if k == pick else ''}" for k, v in enumerate(t))
                 + f" | {100 * (t[pick] / min(t) - 1):.1f} % |")
        print(L[-1], flush=True)
        del a, sa, b, sb, c
    text = "\n".join(L) + "\n"
    if md_path:
        with open(md_path, "w") as f:
            f.write(text)
    return 0


SPLIT_SHAPES = [(1024, 1024, 1024), (16384, 512, 4096), (512, 4096, 4096), (1024, 1024, 4096),
                (1024, 1024, 8192), (1024, 1024, 32768), (512, 512, 16384), (2048, 2048, 16384),
                (4096, 1024, 8192)]


def split_sweep(md_path=None):
    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg
    from tiled_dense_gemm_04_amd.measure import timed_trials

    stream = torch.cuda.Stream()
    names = {i: c["name"] for i, c in enumerate(tg.configs())}
    split_cfgs = [i for i, c in enumerate(tg.configs()) if c["layouts"] == 0xF and not c["generic"]
                  and c["block_m"] == c["block_n"]]
    lines = ["| M x N x K | gemm_f16 (no split) us | planned (cfg, splits) | "
             + " | ".join(f"{names[c][:9]} x{s}" for c in split_cfgs for s in (1, 2, 4, 8)) + " |",
             "|---|---|---|" + "---|" * (4 * len(split_cfgs))]
    for (M, N, K) in SPLIT_SHAPES:
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=5)
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        base = timed_trials(torch, stream, lambda i: tg.gemm_f16(a, b, c, relu=True, stream=stream),
                            trials=5)["median_us"]
        plan = tg.tgemm_split_plan(False, False, M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N)
        cells = []
        for cfg in split_cfgs:
            d = tg.tgemm_config_desc(cfg)
            tiles = -(-M // d["block_m"]) * -(-N // d["block_n"])
            nk = -(-K // d["block_k"])
            for sp in (1, 2, 4, 8):
                if sp > nk or tiles > 1024:
                    cells.append("-")
                    continue
                t = timed_trials(torch, stream, lambda i: tg.gemm_f16_ws(a, b, c, relu=True, stream=stream,
                                                                       cfg=cfg, splits=sp), trials=5)["median_us"]
                cells.append(f"{t:.1f}")
        row = f"| {M}x{N}x{K} | {base:.1f} | {names[plan[0]][:9]}, {plan[1]} | " + " | ".join(cells) + " |"
        print(row, flush=True)
        lines.append(row)
        del a, b, c
        torch.cuda.empty_cache()
    md = "\n".join(lines) + "\n"
    if md_path:
        with open(md_path, "w") as f:
            f.write(md)
    return 0


# Shapes the selector's cost model is fitted on (A and B as given): grid sizes from under
# one round of 256 workgroups to several, K from 512 to 8192.
TABLE_SHAPES = [
    (1024, 1024, 4096), (1536, 1536, 4096), (2048, 2048, 4096), (2560, 2560, 4096), (2048, 4096, 4096),
    (16384, 512, 4096), (3072, 3072, 4096), (3072, 4096, 4096), (4096, 4096, 4096), (5120, 4096, 4096),
    (6144, 6144, 4096), (4096, 8192, 4096), (8192, 8192, 4096),
    (3584, 3584, 2048), (4096, 2560, 2048), (2048, 2048, 2048), (6144, 4096, 2048), (8192, 8192, 2048),
    (4095, 3000, 1000), (4096, 3072, 1024), (1024, 1024, 1024), (2048, 2048, 1024), (4096, 4096, 1024),
    (8192, 8192, 1024), (1024, 1024, 8192), (2048, 2048, 8192), (4096, 4096, 8192), (8192, 8192, 8192),
    (4096, 4096, 512), (8192, 8192, 512), (2560, 5120, 2048), (5120, 5120, 1024),
    (1024, 2048, 4096), (2048, 1024, 2048), (2048, 2048, 16384), (4096, 1024, 8192), (1024, 1024, 16384),
    (3072, 2048, 8192),
]
ROUND = 256  # workgroups in flight at once: one per compute unit


def model_features(tiles: int, K: int):
    R = -(-tiles // ROUND)
    O = tiles / ROUND
    k = K / 1024.0
    return [R, R * k, O, k * O]


def fit_model(rows):
    """rows: [(tiles, K, us)]. Non-negative coefficients (a, b, c, d) minimising the
    relative error of a*R + b*R*k + c*O + d*k*O against us."""
    import numpy as np
    from scipy.optimize import nnls

    X = np.array([model_features(t, K) for t, K, _ in rows], dtype=np.float64)
    y = np.array([us for _, _, us in rows], dtype=np.float64)
    coef, _ = nnls(X / y[:, None], np.ones_like(y))
    return [float(v) for v in coef]


def predict(coef, tiles, K):
    return sum(c * f for c, f in zip(coef, model_features(tiles, K)))


def table_sweep(out_inc, md_path=None, refit=None):
    """Time (or reload) the product configs on TABLE_SHAPES and the workloads, fit the cost
    model and write the selector's table."""
    if refit:
        with open(refit) as f:
            data = json.load(f)
        data = product_only(data)
    else:
        data = measure_table()
        with open(os.path.splitext(out_inc)[0] + ".json", "w") as f:
            json.dump(data, f, indent=1)
    text_inc, text_md = render_table(data)
    with open(out_inc, "w") as f:
        f.write(text_inc)
    if md_path:
        with open(md_path, "w") as f:
            f.write(text_md)
    print(text_md)
    return 0


# Split-K options the table sweep times (gemm_f16_ws_cfg): every split-capable product
# config (all four layouts compiled) at 2, 4 and 8 splits, where the split launch stays
# within one round of workgroups (tiles x splits <= 256, which also bounds the partial
# tiles to what the allocation-free entry point's static scratch holds) and every split
# keeps at least 64 k-tiles.
SPLIT_COUNTS = (2, 4, 8)
SPLIT_MIN_KTILES = 64


def split_options(cfgs, built, M, N, K):
    out = []
    for i in built:
        c = cfgs[i]
        if c["layouts"] != 0xF:
            continue
        tiles = -(-M // c["block_m"]) * -(-N // c["block_n"])
        nk = -(-K // c["block_k"])
        out += [(i, s) for s in SPLIT_COUNTS if tiles * s <= ROUND and nk // s >= SPLIT_MIN_KTILES]
    return out


def product_only(data):
    """Saved timings restricted to the configs the product library compiles now (a config
    demoted to the tooling build since the timings were taken drops out of the exact
    entries and the model; one promoted since then has no timings and needs a new sweep)."""
    import tiled_dense_gemm_04_amd as tg

    built = {"f16": {str(i) for i, c in enumerate(tg.configs()) if c["built"] and not c["generic"]},
             "fp8": {str(i) for i in range(tg.tgemm_fp8_num_configs()) if tg.tgemm_fp8_config_desc(i)["built"]}}
    for kind in ("f16", "fp8"):
        d = data[kind]
        d["configs"] = {i: n for i, n in d["configs"].items() if i in built[kind]}
        for c in d["cases"]:
            c["us"] = {i: v for i, v in c["us"].items() if i in built[kind]}
        d["cases"] = [c for c in d["cases"] if c["us"]]
    for c in data.get("split", {}).get("cases", []):
        c["us"] = {k: v for k, v in c["us"].items() if k.split("x")[0] in built["f16"]}
    return data


def measure_table():
    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg
    from tiled_dense_gemm_04_amd.measure import timed_trials

    stream = torch.cuda.current_stream()
    cfgs = tg.configs()
    f16 = [i for i, c in enumerate(cfgs) if c["built"] and not c["generic"]]
    cases = [(0, M, N, K) for (M, N, K) in TABLE_SHAPES]
    for w in list(W.WORKLOADS.values()) + list(W.LAYOUT_WORKLOADS.values()) + list(W.SPLIT_WORKLOADS.values()):
        case = (2 * int(w.trans_a) + int(w.trans_b), w.M, w.N, w.K)
        if case not in cases:
            cases.append(case)
    data = {"device": torch.cuda.get_device_name(0), "round": ROUND,
            "f16": {"configs": {str(i): cfgs[i]["name"] for i in f16}, "cases": []},
            "fp8": {"configs": {}, "cases": []}, "split": {"cases": []}}
    for (layout, M, N, K) in cases:
        ta, tb = bool(layout & 2), bool(layout & 1)
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=5)
        a = torch.from_numpy(A.T.copy() if ta else A).cuda()
        b = torch.from_numpy(B.T.copy() if tb else B).cuda()
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        times = {}
        for i in f16:
            if not (cfgs[i]["layouts"] >> layout) & 1:
                continue
            times[str(i)] = round(timed_trials(
                torch, stream, lambda j, i=i: tg.gemm_f16_ex(a, b, c, trans_a=ta, trans_b=tb, cfg=i),
                trials=5, warm_ms=30.0)["median_us"], 2)
        best = min(times, key=times.get)
        data["f16"]["cases"].append({"layout": layout, "M": M, "N": N, "K": K, "us": times})
        print(f"f16 layout {layout} {M}x{N}x{K}: " + ", ".join(f"{k}:{v}" for k, v in times.items())
              + f" -> best {best}", flush=True)
        opts = split_options(cfgs, f16, M, N, K)
        if opts:
            ws = tg.workspace_for(max(tg.tgemm_workspace_bytes_cfg(i, s, M, N) for i, s in opts), a.device,
                                  stream.cuda_stream)
            stimes = {f"{i}x{s}": round(timed_trials(
                torch, stream, lambda j, i=i, s=s: tg.gemm_f16_ws(a, b, c, trans_a=ta, trans_b=tb, cfg=i, splits=s,
                                                                  workspace=ws),
                trials=5, warm_ms=30.0)["median_us"], 2) for i, s in opts}
            data["split"]["cases"].append({"layout": layout, "M": M, "N": N, "K": K, "us": stimes})
            print(f"split layout {layout} {M}x{N}x{K}: " + ", ".join(f"{k}:{v}" for k, v in stimes.items()),
                  flush=True)
            del ws
        del a, b, c
        torch.cuda.empty_cache()
    nf8 = tg.tgemm_fp8_num_configs()
    f8 = [i for i in range(nf8) if tg.tgemm_fp8_config_desc(i)["built"]]
    data["fp8"]["configs"] = {str(i): tg.tgemm_fp8_config_desc(i)["name"] for i in f8}
    f8cases = [(M, N, K) for (M, N, K) in TABLE_SHAPES if N % 8 == 0 and K % 16 == 0]
    for w in W.FP8_WORKLOADS.values():
        if (w.M, w.N, w.K) not in f8cases:
            f8cases.append((w.M, w.N, w.K))
    for (M, N, K) in f8cases:
        A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=5)
        a, sa, b, sb = (torch.from_numpy(x).cuda() for x in (A, SA, B, SB))
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        times = {str(i): round(timed_trials(
            torch, stream, lambda j, i=i: tg.gemm_fp8_block(a, sa, b, sb, c, cfg=i),
            trials=5, warm_ms=30.0)["median_us"], 2) for i in f8}
        data["fp8"]["cases"].append({"layout": 0, "M": M, "N": N, "K": K, "us": times})
        print(f"fp8 {M}x{N}x{K}: " + ", ".join(f"{k}:{v}" for k, v in times.items()), flush=True)
        del a, sa, b, sb, c
        torch.cuda.empty_cache()
    return data


def _tiles(name: str, M: int, N: int) -> int:
    """Workgroups of a config from its name (kind letter, then BMxBNxBK)."""
    bm, bn = (int(v) for v in name[1:].split("_")[0].split("x")[:2])
    return -(-M // bm) * -(-N // bn)


def render_table(data):
    """(C++ table, markdown report) from measured timings."""
    L_inc = ["// tgemm_choice.inc -- the config selector's table, generated by",
             "// `python -m tiled_dense_gemm_04_amd.sweep --write-table` from timings on "
             f"{data['device']}; do not edit by hand.",
             "// Exact entries: every shape the sweep timed, with its fastest product config.",
             "// Model entries: per product config, microseconds ~ a*R + b*R*k + c*O + d*k*O with",
             f"// R = ceil(tiles / {data['round']}), O = tiles / {data['round']}, k = K / 1024 (tiles = the config's",
             "// workgroup count); non-negative least squares on relative error over the timed",
             "// shapes with A and B as given."]
    L_md = ["# Config selector table: timings, fitted cost model, choice quality (one MI355X)", "",
            "Command (from the repository root): `python -m tiled_dense_gemm_04_amd.sweep --write-table "
            "tiled_dense_gemm_04_amd/csrc/tgemm_choice.inc --md out/config_choice.md`", "",
            f"Device: {data['device']}. Every product config on every shape: 10 warm-up calls and >= 30 ms",
            "of calls, then 5 trials of >= 20 ms (HIP events), median microseconds per call. The",
            "selector takes an exact entry when the shape was timed, else the cost model's argmin;",
            "`held-out loss` is the loss of the model's pick when that shape is left out of the fit",
            "(the model alone, as for a shape the sweep never saw).", ""]
    for kind, label in (("f16", "fp16 GEMM (+ ReLU), N(0,1) inputs"),
                        ("fp8", "fp8 block-scaled GEMM (E4M3 codes, 1 x 128 / 128 x 128 scales)")):
        d = data[kind]
        names = d["configs"]
        ids = sorted(names, key=int)
        cases = d["cases"]
        fit_rows = {i: [(_tiles(names[i], c["M"], c["N"]), c["K"], c["us"][i]) for c in cases
                        if c["layout"] == 0 and i in c["us"]] for i in ids}
        coefs = {i: fit_model(fit_rows[i]) for i in ids}
        prefix = "kF16" if kind == "f16" else "kFp8"
        L_inc += ["", f"static const ChoiceExact {prefix}Exact[] = {{"]
        for c in cases:
            best = min(c["us"], key=c["us"].get)
            L_inc.append(f"    {{{c['layout']}, {c['M']}, {c['N']}, {c['K']}, {best}}},")
        L_inc += ["};", f"static const ChoiceModel {prefix}Model[] = {{"]
        for i in ids:
            a, b, cc, dd = coefs[i]
            L_inc.append(f"    {{{i}, {a:.6g}, {b:.6g}, {cc:.6g}, {dd:.6g}}},  // {names[i]}")
        L_inc.append("};")
        # report
        L_md += [f"## {label}", "",
                 "| layout | M x N x K | " + " | ".join(names[i] for i in ids)
                 + " | fastest | model pick | held-out pick | held-out loss |",
                 "|---|---|" + "---|" * (len(ids) + 4)]
        losses = []
        for n, c in enumerate(cases):
            best = min(c["us"], key=c["us"].get)
            avail = [i for i in ids if i in c["us"]]
            pick = min(avail, key=lambda i: predict(coefs[i], _tiles(names[i], c["M"], c["N"]), c["K"]))
            held = {i: fit_model([r for m, r in enumerate(
                [(_tiles(names[i], x["M"], x["N"]), x["K"], x["us"].get(i)) for x in cases]) if m != n
                and cases[m]["layout"] == 0 and r[2] is not None]) for i in avail}
            hpick = min(avail, key=lambda i: predict(held[i], _tiles(names[i], c["M"], c["N"]), c["K"]))
            loss = 100 * (c["us"][hpick] / c["us"][best] - 1)
            losses.append(loss)
            L_md.append(f"| {c['layout']} | {c['M']}x{c['N']}x{c['K']} | "
                        + " | ".join(("**%.1f**" if i == best else "%.1f") % c["us"][i] if i in c["us"] else "-"
                                     for i in ids)
                        + f" | {names[best]} | {names[pick]} | {names[hpick]} | {loss:.1f} % |")
        L_md += ["", "Fitted coefficients (microseconds):", "",
                 "| config | a (per round) | b (per round per 1024 of K) | c (per round's worth of tiles) | d (per round's worth of tiles per 1024 of K) | median abs. rel. error |",
                 "|---|---|---|---|---|---|"]
        for i in ids:
            errs = sorted(abs(predict(coefs[i], t, K) / us - 1) for t, K, us in fit_rows[i])
            med = errs[len(errs) // 2] if errs else float("nan")
            L_md.append(f"| {names[i]} | " + " | ".join(f"{v:.3f}" for v in coefs[i]) + f" | {100 * med:.1f} % |")
        losses.sort()
        L_md += ["", f"Held-out loss over {len(losses)} shapes: median {losses[len(losses) // 2]:.1f} %, "
                 f"mean {sum(losses) / len(losses):.1f} %, max {losses[-1]:.1f} %.", ""]
    inc_split, md_split = render_split(data)
    return "\n".join(L_inc + inc_split) + "\n", "\n".join(L_md + md_split) + "\n"


def render_split(data):
    """The split-K part of the table: per timed shape with split options, the fastest of
    the unsplit default (the f16 exact entry) and the timed splits, as (cfg, splits); cfg
    -1 with 1 split means the unsplit default."""
    names = data["f16"]["configs"]
    unsplit = {(c["layout"], c["M"], c["N"], c["K"]): c["us"] for c in data["f16"]["cases"]}
    inc = ["", "// Split-K plan (gemm_f16_ws): every shape the sweep timed split options on, with the",
           "// fastest of the unsplit choice (cfg -1, 1 split) and the timed (cfg, splits).",
           "static const SplitExact kSplitExact[] = {"]
    md = ["## split-K plan (gemm_f16_ws), the same inputs", "",
          "Options: every split-capable product config at 2, 4 and 8 splits with tiles x splits <= 256 and at",
          "least 64 k-tiles per split. `unsplit` is the fastest config without splitting (the table's",
          "choice for gemm_f16). Shapes not listed take the fixed rule in tgemm_api.cpp.", "",
          "| layout | M x N x K | unsplit us | split options us | plan |", "|---|---|---|---|---|"]
    rows = 0
    for c in data.get("split", {}).get("cases", []):
        key = (c["layout"], c["M"], c["N"], c["K"])
        if not c["us"] or key not in unsplit:
            continue
        base = min(unsplit[key].values())
        best = min(c["us"], key=c["us"].get)
        cfg, splits = (int(best.split("x")[0]), int(best.split("x")[1])) if c["us"][best] < base else (-1, 1)
        inc.append(f"    {{{c['layout']}, {c['M']}, {c['N']}, {c['K']}, {cfg}, {splits}}},")
        opts = ", ".join(f"{names[k.split('x')[0]]} x{k.split('x')[1]}: " + ("**%.1f**" if k == best and cfg >= 0
                                                                             else "%.1f") % v
                         for k, v in c["us"].items())
        plan = f"{names[str(cfg)]} x{splits}" if cfg >= 0 else "no split"
        md.append(f"| {c['layout']} | {c['M']}x{c['N']}x{c['K']} | {base:.1f} | {opts} | {plan} |")
        rows += 1
    if rows == 0:  # (a C++ array needs an element)
        inc.append("    {-1, 0, 0, 0, -1, 1},")
    inc.append("};")
    md.append("")
    return inc, md


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--iters", type=int, default=30)
    ap.add_argument("--workloads", default=None, help="comma-separated names (default: all)")
    ap.add_argument("--torch", action="store_true",
                    help="also time torch.matmul (+ relu) on the same inputs, as context only")
    ap.add_argument("--split", action="store_true", help="split-K sweep on small-grid shapes")
    ap.add_argument("--choice", action="store_true", help="default config choice against the candidates")
    ap.add_argument("--md", default=None, help="write the table (markdown) here")
    ap.add_argument("--write-table", default=None, metavar="INC",
                    help="time the product configs, fit the selector's cost model, write its table here")
    ap.add_argument("--refit", default=None, metavar="JSON",
                    help="with --write-table: refit from saved timings instead of timing (no GPU)")
    args = ap.parse_args()
    if args.write_table:
        return table_sweep(args.write_table, args.md, args.refit)
    if args.split:
        return split_sweep(args.md)
    if args.choice:
        return choice_sweep(args.md)

    import torch

    import tgemm_workloads as W
    import tiled_dense_gemm_04_amd as tg

    works = [W.HEADLINE] + list(W.WORKLOADS.values())
    if args.workloads:
        keep = set(args.workloads.split(","))
        works = [w for w in works if w.name in keep]
    cfgs = tg.configs()
    results = []
    for w in works:
        A, B = w.inputs()
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B).cuda()
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        default = tg.tgemm_select_config(w.M, w.N, w.K, a.data_ptr(), a.stride(0), b.data_ptr(),
                                         b.stride(0), c.data_ptr(), c.stride(0))
        row = {"workload": w.name, "default_cfg": default, "times_us": {}}
        for i, cd in enumerate(cfgs):
            us = time_config(tg, torch, a, b, c, w.relu, i, args.iters)
            tf = w.flop / (us * 1e-6) / 1e12
            row["times_us"][cd["name"]] = round(us, 2)
            print(f"{w.name:28s} cfg {i} {cd['name']:30s} {us:9.2f} us {tf:8.1f} TFLOP/s "
                  f"({100 * tf / PEAK_TFLOPS:5.1f} %){' <- default' if i == default else ''}", flush=True)
        if args.torch:
            def tmm():
                r = torch.matmul(a, b)
                return torch.relu_(r) if w.relu else r
            for _ in range(5):
                tmm()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.iters):
                tmm()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / args.iters * 1e3
            tf = w.flop / (us * 1e-6) / 1e12
            row["torch_matmul_us"] = round(us, 2)
            print(f"{w.name:28s} torch.matmul{'+relu' if w.relu else ''} (context) {us:9.2f} us {tf:8.1f} TFLOP/s "
                  f"({100 * tf / PEAK_TFLOPS:5.1f} %)", flush=True)
        best = min(row["times_us"], key=row["times_us"].get)
        row["best"] = best
        results.append(row)
        del a, b, c
        torch.cuda.empty_cache()
    if args.out:
        with open(args.out, "w") as f:
            json.dump(results, f, indent=1)
    if args.md:
        with open(args.md, "w") as f:
            f.write(sweep_markdown(results, cfgs, args, torch.cuda.get_device_name(0)))
    return 0


def sweep_markdown(results, cfgs, args, device) -> str:
    """Configs as rows, workloads as columns, the fastest per column in bold."""
    from bench import kernel_source_hash

    names = [cd["name"] for cd in cfgs]
    cmd = "python -m tiled_dense_gemm_04_amd.sweep" + (" --torch" if args.torch else "") + \
        f" --iters {args.iters} --md out/sweep.md"
    L = ["# Config sweep, all measured workloads (one MI355X)", "",
         f"Command (from the repository root): `{cmd}`", "",
         f"Device: {device}. Every table config on every workload: {args.iters} timed launches after 5",
         "warm-up, HIP events, microseconds per launch; **bold** is the fastest config per workload.",
         "`torch.matmul` (+ `relu_`) is hipBLASLt on the same inputs, context only. Absolute times vary",
         "by ~5-10 % between MI355X boxes (power and thermal state); compare within a column.",
         "Configs marked (t) are sweep-only variants, timed on the tooling build (libtgemm_stamps.so);",
         f"the rest run on the product library. Kernel source hash {kernel_source_hash()}.", "",
         "| config | " + " | ".join(r["workload"] for r in results) + " |",
         "|---|" + "---|" * len(results)]
    for n in names:
        cells = []
        for r in results:
            t = r["times_us"].get(n)
            cells.append("-" if t is None else (f"**{t:.2f}**" if n == r["best"] else f"{t:.2f}"))
        L.append(f"| {n}{'' if cfgs[names.index(n)]['built'] else ' (t)'} | " + " | ".join(cells) + " |")
    if any("torch_matmul_us" in r for r in results):
        L.append("| torch.matmul(+relu) | " + " | ".join(f"{r['torch_matmul_us']:.2f}" if "torch_matmul_us" in r
                                                        else "-" for r in results) + " |")
    L += ["", "Default choice per workload (the config `gemm_f16` picks): " +
          ", ".join(f"{r['workload']} -> {names[r['default_cfg']] if r['default_cfg'] >= 0 else 'generic'}"
                    for r in results) + "."]
    return "\n".join(L) + "\n"


if __name__ == "__main__":
    sys.exit(main())
