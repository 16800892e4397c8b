"""The host logic of libtgemm (tgemm_api.cpp: argument checks, config selection, split-K
plans and workspace sizes, grouped batching, the fp8 and quantizer entry points) compiled
for the CPU under AddressSanitizer and UndefinedBehaviorSanitizer, with recording stubs in
place of the kernels and the HIP runtime (tests/host_sanitize/). The driver checks every
return code against the header's argument rules and every recorded launch against its
arguments; the sanitizers stop it on any out-of-bounds access, overflow or other undefined
behaviour. The stub config tables are rebuilt from the same lists as the library's and
compared with the built library here."""
import os
import shutil
import subprocess

import pytest

import tiled_dense_gemm_04_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CXX = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def driver_output(tmp_path_factory):
    if not os.path.exists(CXX):
        pytest.skip("clang++ of the ROCm toolchain not found")
    exe = str(tmp_path_factory.mktemp("host_sanitize") / "driver")
    cmd = [CXX, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc"),
           "-I" + HERE, os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc", "tgemm_api.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "6000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_host_logic_under_sanitizers(driver_output):
    last = driver_output.strip().splitlines()[-1]
    assert last.startswith("host logic ok"), last
    checks = int(last.split(":")[1].split()[0])
    launches = int(last.split(",")[1].split()[0])
    assert checks > 50000 and launches > 3000, last


def test_stub_tables_match_library(driver_output):
    rows = [ln.split() for ln in driver_output.splitlines() if ln.startswith("cfg ")]
    assert len(rows) == tg.tgemm_num_configs()
    for r, c in zip(rows, tg.configs()):
        vals = [int(v) for v in r[2:14]]
        want = [c[k] for k in ("block_m", "block_n", "block_k", "stages", "waves_m", "waves_n", "panel",
                               "xcd_remap", "generic", "layouts", "built", "lds_bytes")]
        assert vals == want and r[14] == c["name"], (r, c)
    rows8 = [ln.split() for ln in driver_output.splitlines() if ln.startswith("fp8 ")]
    assert len(rows8) == tg.tgemm_fp8_num_configs()
    for r, c in zip(rows8, tg.fp8_configs()):
        vals = [int(v) for v in r[2:11]]
        want = [c[k] for k in ("block_m", "block_n", "block_k", "stages", "waves_m", "waves_n", "panel",
                               "xcd_remap", "built")]
        assert vals == want and r[11] == c["name"], (r, c)
