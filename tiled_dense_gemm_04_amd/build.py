"""Build libtgemm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and two twins
from the same sources: the tooling build libtgemm_stamps.so (per-workgroup timestamps,
every config row of tgemm_configs.h compiled, including the sweep-only variants, and the
MFMA throughput probe; used only by the measurement tools) and the debugging build
libtgemm_debugfill.so (TGEMM_DEBUG_FILL: every LDS copy destination is overwritten with
NaN bytes before the copy is issued; used only by its GPU test).

Usage: python -m tiled_dense_gemm_04_amd.build   (always recompiles both)
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libtgemm.so")
STAMPS_LIBRARY = os.path.join(PKG, "libtgemm_stamps.so")
DEBUGFILL_LIBRARY = os.path.join(PKG, "libtgemm_debugfill.so")
VARIANTS = {
    "product": (LIBRARY, []),
    "stamps": (STAMPS_LIBRARY, ["-DTGEMM_STAMPS", "-DTGEMM_SWEEP_CONFIGS"]),
    "debugfill": (DEBUGFILL_LIBRARY, ["-DTGEMM_DEBUG_FILL"]),
}
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "tgemm_kernels.hip"), os.path.join(CSRC, "tgemm_fp8.hip"),
           os.path.join(CSRC, "tgemm_api.cpp")]

# Device code: gfx950 only. Packed-fp32 instruction selection is switched off for all
# device code; -fvisibility=hidden keeps everything but the TGEMM_API entry points local.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    # the LDS-DMA inline asm clobbers M0 on purpose (see dma_to_lds)
    "-Wno-inline-asm",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtgemm)")


RESOURCES = os.path.join(PKG, "kernel_resources.txt")


def kernel_resources(remarks: str) -> dict:
    """{kernel: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, name = {}, None
    for ln in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][\w \[\]/]*?): (\S+) \[-Rpass-analysis", ln)
        if m and name:
            out[name][m.group(1).strip()] = m.group(2)
    return out


def check_resources(res: dict) -> list:
    """Kernels that use scratch memory or spill: a missed unroll or a spill in a hot loop
    turns register arrays into scratch loads and serializes the copy stream."""
    bad = []
    for k, f in res.items():
        if f.get("ScratchSize [bytes/lane]", "0") != "0" or f.get("VGPRs Spill", "0") != "0" or \
                f.get("SGPRs Spill", "0") != "0":
            bad.append(k)
    return bad


def build(verbose: bool = False, extra_flags=None, stamps: bool = False, variant: str | None = None) -> str:
    """Compile one variant. The product build also records every kernel's registers,
    scratch and LDS (kernel_resources.txt) and fails if any kernel uses scratch memory."""
    variant = variant or ("stamps" if stamps else "product")
    target, vflags = VARIANTS[variant]
    tmp = target + ".tmp"
    flags = list(extra_flags or []) + vflags
    if variant == "product":
        flags.append("-Rpass-analysis=kernel-resource-usage")
    cmd = [hipcc()] + HIPCC_FLAGS + flags + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    noise = "is not a recognized feature for this target"
    out = r.stdout + r.stderr
    msgs = [ln for ln in out.splitlines() if noise not in ln and "-Rpass-analysis" not in ln and
            not re.match(r"^\s*(\d+ \|.*|\|\s*\^)$", ln)]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    if variant == "product":
        res = kernel_resources(out)
        with open(RESOURCES, "w") as f:
            for k in sorted(res):
                f.write(k + " " + " ".join(f"{a}={b}" for a, b in res[k].items()) + "\n")
        bad = check_resources(res)
        if bad:
            os.remove(tmp)
            raise RuntimeError("kernels use scratch memory or spill registers:\n" + "\n".join(bad))
    os.replace(tmp, target)
    return target


def build_all(verbose: bool = False):
    """All three libraries, compiled in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(len(VARIANTS)) as ex:
        futs = [ex.submit(build, verbose, None, False, v) for v in VARIANTS]
        return [f.result() for f in futs]


if __name__ == "__main__":
    for path in build_all(verbose=True):
        print(path)
    sys.exit(0)
