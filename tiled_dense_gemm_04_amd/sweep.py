"""Offline config sweep: time every applicable table config of libtgemm on the measured
workloads and report the fastest per workload (the evidence behind the config choice in
tgemm_api.cpp's choose_fast). With --split, time split-K instead: the 256 x 256 and
128 x 128 ping-pong configs at 1, 2, 4 and 8 splits per output tile on small-grid shapes
(the evidence behind split_plan). Needs a GPU.

  python -m tiled_dense_gemm_04_amd.sweep [--out results.json] [--md out.md] [--torch] [--iters 30]
  python -m tiled_dense_gemm_04_amd.sweep --split [--md out.md]
  python -m tiled_dense_gemm_04_amd.sweep --choice [--md out.md]

--choice checks the default config choice (fp16 choose_fast, fp8 fp8_choose) against the
candidate configs on shapes from 1024^2 to 6144^2, timed with the measurement protocol.
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


def time_config(tg, torch, a, b, c, relu, cfg, iters, warmup=5):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        tg.gemm_f16(a, b, c, relu=relu, cfg=cfg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        tg.gemm_f16(a, b, c, relu=relu, cfg=cfg)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3  # us


CHOICE_SHAPES = [(1024, 1024, 4096), (1536, 1536, 4096), (2048, 2048, 4096), (2560, 2560, 4096),
                 (2048, 4096, 4096), (16384, 512, 4096), (3072, 3072, 4096), (3584, 3584, 2048),
                 (4096, 2560, 2048), (4095, 3000, 1000), (4096, 3072, 1024), (3072, 4096, 4096),
                 (5120, 4096, 4096), (6144, 6144, 4096)]
CHOICE_F16 = ["p128x128x64_s2_w2x2_p4_x1", "m128x128x32_s4_w2x4_p4_x1", "m256x128x32_s4_w2x4_p4_x1",
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
         "gpurun_out/choice.md`", "",
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


SPLIT_SHAPES = [(1024, 1024, 1024), (16384, 512, 4096), (512, 4096, 4096), (1024, 1024, 32768),
                (512, 512, 16384), (2048, 2048, 16384), (4096, 1024, 8192)]


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
    args = ap.parse_args()
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
            f.write(sweep_markdown(results, [cd["name"] for cd in cfgs], args, torch.cuda.get_device_name(0)))
    return 0


def sweep_markdown(results, names, args, device) -> str:
    """Configs as rows, workloads as columns, the fastest per column in bold."""
    cmd = "python -m tiled_dense_gemm_04_amd.sweep" + (" --torch" if args.torch else "") + \
        f" --iters {args.iters} --md gpurun_out/sweep.md"
    L = ["# Config sweep, all measured workloads (one MI355X)", "",
         f"Command (from the repository root): `{cmd}`", "",
         f"Device: {device}. Every table config on every workload: {args.iters} timed launches after 5",
         "warm-up, HIP events, microseconds per launch; **bold** is the fastest config per workload.",
         "`torch.matmul` (+ `relu_`) is hipBLASLt on the same inputs, context only. Absolute times vary",
         "by ~5-10 % between MI355X boxes (power and thermal state); compare within a column.", "",
         "| config | " + " | ".join(r["workload"] for r in results) + " |",
         "|---|" + "---|" * len(results)]
    for n in names:
        cells = []
        for r in results:
            t = r["times_us"].get(n)
            cells.append("-" if t is None else (f"**{t:.2f}**" if n == r["best"] else f"{t:.2f}"))
        L.append(f"| {n} | " + " | ".join(cells) + " |")
    if any("torch_matmul_us" in r for r in results):
        L.append("| torch.matmul(+relu) | " + " | ".join(f"{r['torch_matmul_us']:.2f}" if "torch_matmul_us" in r
                                                        else "-" for r in results) + " |")
    L += ["", "Default choice per workload (the config `gemm_f16` picks): " +
          ", ".join(f"{r['workload']} -> {names[r['default_cfg']] if r['default_cfg'] >= 0 else 'generic'}"
                    for r in results) + "."]
    return "\n".join(L) + "\n"


if __name__ == "__main__":
    sys.exit(main())
