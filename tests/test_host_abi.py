"""libtgemm on the CPU: the C-ABI library loads and exports every symbol the header
declares; argument validation, error codes, config selection and the workgroup -> tile
map are checked without any GPU work (every call here returns before touching HIP)."""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_04_amd as tg
from choice_table import expected_choice, parse_choice_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not (os.path.exists(tg.LIBRARY) and os.path.exists(tg.STAMPS_LIBRARY)):
        from tiled_dense_gemm_04_amd import build
        build.build_all()
    tg.lib()
    tg.stamps_lib()


def header_symbols(name="tgemm.h"):
    text = open(os.path.join(ROOT, "include", name)).read()
    text = text.replace("#define TGEMM_API __attribute__((visibility(\"default\")))", "")
    return sorted(set(re.findall(r"^TGEMM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def exported(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    return {n for n in names if n.startswith(("gemm_", "tgemm_", "quant_"))}


def test_exports_every_header_symbol():
    syms = header_symbols()
    assert len(syms) == 26, syms
    assert sorted(tg.EXPORTS) == syms
    L = tg.lib()
    for s in syms:
        assert hasattr(L, s), s


def test_only_header_symbols_are_exported():
    assert exported(tg.LIBRARY) == set(header_symbols())


def test_instrumented_build_exports():
    """libtgemm_stamps.so exports tgemm.h plus tgemm_stamps.h, and nothing else."""
    extra = header_symbols("tgemm_stamps.h")
    assert sorted(tg.STAMPS_EXPORTS) == extra
    assert exported(tg.STAMPS_LIBRARY) == set(header_symbols()) | set(extra)
    assert not (exported(tg.LIBRARY) & set(extra))
    S = tg.stamps_lib()
    import ctypes
    nwg, words = ctypes.c_int(), ctypes.c_int()
    assert S.tgemm_stamps_capacity(ctypes.byref(nwg), ctypes.byref(words)) == tg.TGEMM_OK
    text = open(os.path.join(ROOT, "include", "tgemm_stamps.h")).read()
    assert f"#define TGEMM_STAMP_WORKGROUPS {nwg.value}" in text
    assert f"#define TGEMM_STAMP_WORDS {words.value}" in text
    assert S.tgemm_stamps_capacity(None, ctypes.byref(words)) == tg.TGEMM_ENULL
    assert S.tgemm_stamps_read(None, 8) == tg.TGEMM_ENULL
    buf = (ctypes.c_uint64 * 8)()
    assert S.tgemm_stamps_read(buf, -1) == tg.TGEMM_EINVAL_DIM
    assert S.tgemm_stamps_read(buf, nwg.value * words.value + 1) == tg.TGEMM_EINVAL_DIM


def test_probe_argument_checks():
    """Rejected before any HIP call; the shape constants match the header."""
    L = tg.stamps_lib()
    text = open(os.path.join(ROOT, "include", "tgemm_stamps.h")).read()
    assert f"#define TGEMM_PROBE_THREADS {tg.PROBE_THREADS}" in text
    assert f"#define TGEMM_PROBE_MFMA_PER_ITER {tg.PROBE_MFMA_PER_ITER}" in text
    assert L.tgemm_mfma_probe(1, 1, None, None) == tg.TGEMM_ENULL
    assert L.tgemm_mfma_probe(0, 1, 16, None) == tg.TGEMM_EINVAL_DIM
    assert L.tgemm_mfma_probe((1 << 20) + 1, 1, 16, None) == tg.TGEMM_EINVAL_DIM
    assert L.tgemm_mfma_probe(1, 0, 16, None) == tg.TGEMM_EINVAL_DIM
    assert L.tgemm_mfma_probe(1, (1 << 24) + 1, 16, None) == tg.TGEMM_EINVAL_DIM
    for name, mode in tg.PROBE_MODES.items():
        macro = {"synthetic": "SYNTHETIC", "operands": "OPERANDS", "operands_32x32": "OPERANDS_32",
                 "lds_reads": "LDS_READS"}[name]
        assert f"#define TGEMM_PROBE_{macro} {mode}" in text
    P = L.tgemm_mfma_probe_ex
    assert P(-1, 1, 1, 16, 16, None) == tg.TGEMM_EINVAL_DIM
    assert P(len(tg.PROBE_MODES), 1, 1, 16, 16, None) == tg.TGEMM_EINVAL_DIM
    assert P(0, 1, 1, None, None, None) == tg.TGEMM_ENULL
    for mode in (1, 2, 3):
        assert P(mode, 1, 1, None, 16, None) == tg.TGEMM_ENULL      # operands needed
        assert P(mode, 1, 1, 24, 16, None) == tg.TGEMM_EALIGN       # 16-byte aligned operands
        assert P(mode, 0, 1, 16, 16, None) == tg.TGEMM_EINVAL_DIM
        assert P(mode, 1, (1 << 24) + 1, 16, 16, None) == tg.TGEMM_EINVAL_DIM


def test_error_codes_match_header():
    text = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    codes = dict((m.group(1), int(m.group(2)))
                 for m in re.finditer(r"#define (TGEMM_E\w+|TGEMM_OK)\s+\(?(-?\d+)\)?", text))
    for name, val in codes.items():
        assert getattr(tg, name) == val, name
    for val in codes.values():
        assert tg.tgemm_strerror(val) != "unknown error code"
    assert tg.tgemm_strerror(12345) == "unknown error code"
    assert "gfx950" in tg.tgemm_version()


def test_config_table():
    n = tg.tgemm_num_configs()
    assert n >= 2
    # the per-config GPU tests are parametrized over these counts
    assert n <= 32
    assert sum(c["layouts"] == 0xF for c in tg.configs()) <= 6
    cfgs = tg.configs()
    assert cfgs[0]["generic"] == 1
    for c in cfgs[1:]:
        assert c["generic"] == 0
        assert c["lds_bytes"] <= 160 * 1024
        # operand tiles sit in LDS at their own extent when it is a multiple of 128 or 192,
        # else rounded up to a multiple of 128
        ext = lambda r: r if r % 128 == 0 or r == 192 else -(-r // 128) * 128
        bm_l, bn_l = ext(c["block_m"]), ext(c["block_n"])
        ring = c["stages"] * (bm_l + bn_l) * c["block_k"] * 2
        # the epilogue stages each wave's tile in rows of a power of two (>= 4) of 16-byte chunks
        cpr = c["block_n"] // c["waves_n"] // 8
        scpr = next(p for p in (4, 8, 16, 32) if p >= cpr)
        staged = c["waves_m"] * c["waves_n"] * (c["block_m"] // c["waves_m"]) * scpr * 16
        assert c["lds_bytes"] == max(ring, staged), c
        assert c["block_m"] % (16 * c["waves_m"]) == 0 and c["block_n"] % (16 * c["waves_n"]) == 0
        assert c["block_n"] >= 128 and c["block_k"] in (16, 32, 64, 128)
        threads = 64 * c["waves_m"] * c["waves_n"]
        # 16-byte copies split evenly over the threads, or with one extra copy for half of them
        for ext_units in (bm_l * c["block_k"] // 8, c["block_k"] * bn_l // 8):
            assert ext_units % threads in (0, threads // 2)
        assert c["name"][1:].startswith("%dx%dx%d" % (c["block_m"], c["block_n"], c["block_k"]))
    with pytest.raises(tg.TgemmError):
        tg.tgemm_config_desc(n)
    with pytest.raises(tg.TgemmError):
        tg.tgemm_config_desc(-1)


def config_list_prod_flags():
    """PROD column of every row of csrc/tgemm_configs.h, in table order (fp16, then fp8)."""
    text = open(os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc", "tgemm_configs.h")).read()
    lists = {}
    for m in re.finditer(r"#define (TGEMM_\w+_CONFIGS)\(X\)((?:[^\n]*\\\n)*[^\n]*)", text):
        lists[m.group(1)] = [int(r.split(",")[-1]) for r in re.findall(r"X\(([^)]*)\)", m.group(2))]
    f16 = [1] + sum((lists[k] for k in ("TGEMM_FAST_CONFIGS", "TGEMM_PIPE_CONFIGS", "TGEMM_PP_CONFIGS",
                                         "TGEMM_PP1_CONFIGS", "TGEMM_QUAD_CONFIGS", "TGEMM_PIPE2_CONFIGS")), [])
    return f16, lists["TGEMM_FP8_CONFIGS"]


def test_built_flags_follow_config_lists():
    """The product library compiles exactly the rows marked PROD (plus the generic kernel);
    the tooling build compiles every row; both list the same rows under the same names."""
    f16, f8 = config_list_prod_flags()
    P, S = tg.lib(), tg.stamps_lib()

    def desc(L, fn, i):
        info = tg.ConfigInfo()
        assert getattr(L, fn)(i, ctypes.byref(info)) == tg.TGEMM_OK
        return info.as_dict()

    assert P.tgemm_num_configs() == S.tgemm_num_configs() == len(f16)
    assert P.tgemm_fp8_num_configs() == S.tgemm_fp8_num_configs() == len(f8)
    for fn, flags in (("tgemm_config_desc", f16), ("tgemm_fp8_config_desc", f8)):
        for i, prod in enumerate(flags):
            p, s = desc(P, fn, i), desc(S, fn, i)
            assert p["built"] == prod and s["built"] == 1, (fn, i)
            assert {k: v for k, v in p.items() if k != "built"} == {k: v for k, v in s.items() if k != "built"}
    # a row the product library does not compile is refused before any HIP call
    off = f16.index(0)
    assert tg.gemm_f16_cfg_raw(off, 256, 256, 256, A16, 256, A16, 256, A16, 256, 1, None) == tg.TGEMM_EINVAL_CFG
    off8 = f8.index(0)
    assert tg.gemm_fp8_block_cfg_raw(off8, 256, 256, 256, A16, 256, A16, A16, 256, A16, A16, 256, 0,
                                     None) == tg.TGEMM_EINVAL_CFG


A16 = 0x100000  # a fake, 16-byte-aligned address; select_config never dereferences


@pytest.mark.parametrize("args,code", [
    ((-1, 8, 8), tg.TGEMM_EINVAL_DIM),
    ((8, -1, 8), tg.TGEMM_EINVAL_DIM),
    ((8, 8, -1), tg.TGEMM_EINVAL_DIM),
    ((1 << 31, 8, 8), tg.TGEMM_EINVAL_DIM),
])
def test_select_rejects_bad_dims(args, code):
    M, N, K = args
    assert tg.tgemm_select_config(M, N, K, A16, max(1, K), A16, max(1, N), A16, max(1, N)) == code


def test_select_rejects_bad_ld_null_align():
    s = tg.tgemm_select_config
    assert s(8, 8, 8, A16, 7, A16, 8, A16, 8) == tg.TGEMM_EINVAL_LD
    assert s(8, 8, 8, A16, 8, A16, 7, A16, 8) == tg.TGEMM_EINVAL_LD
    assert s(8, 8, 8, A16, 8, A16, 8, A16, 7) == tg.TGEMM_EINVAL_LD
    # any ld at or above the row length is valid: operand strides past the fast kernels'
    # 32-bit buffer ranges take the generic kernel, ldc is not limited
    assert s(8, 8, 8, A16, 1 << 22, A16, 8, A16, 8) > 0
    assert s(8, 8, 8, A16, (1 << 22) + 8, A16, 8, A16, 8) == 0
    assert s(8, 8, 8, A16, 8, A16, (1 << 22) + 8, A16, 8) == 0
    assert s(8, 8, 8, A16, 1 << 40, A16, 1 << 40, A16, 8) == 0
    assert s(8, 8, 8, A16, 8, A16, 8, A16, 1 << 40) > 0
    assert tg.tgemm_select_config_ex(1, 1, 8, 8, 8, A16, (1 << 22) + 8, A16, 8, A16, 8) == 0
    assert tg.tgemm_select_config_ex(1, 1, 8, 8, 8, A16, 8, A16, (1 << 22) + 8, A16, 8) == 0
    assert s(8, 8, 8, 0, 8, A16, 8, A16, 8) == tg.TGEMM_ENULL
    assert s(8, 8, 8, A16, 8, 0, 8, A16, 8) == tg.TGEMM_ENULL
    assert s(8, 8, 8, A16, 8, A16, 8, 0, 8) == tg.TGEMM_ENULL
    assert s(8, 8, 8, A16 + 1, 8, A16, 8, A16, 8) == tg.TGEMM_EALIGN
    assert s(8, 8, 8, A16, 8, A16, 8, A16 + 3, 8) == tg.TGEMM_EALIGN
    # empty output: no pointers needed; K == 0: only C is needed
    assert s(0, 8, 8, 0, 8, 0, 8, 0, 8) == tg.SELECT_NOOP
    assert s(8, 0, 8, 0, 8, 0, 1, 0, 1) == tg.SELECT_NOOP
    assert s(8, 8, 0, 0, 1, 0, 8, A16, 8) == tg.SELECT_ZERO_FILL
    assert s(8, 8, 0, 0, 1, 0, 8, 0, 8) == tg.TGEMM_ENULL


def test_select_fast_vs_generic():
    s = tg.tgemm_select_config
    big = s(4096, 4096, 4096, A16, 4096, A16, 4096, A16, 4096)
    assert big > 0 and tg.tgemm_config_desc(big)["generic"] == 0
    # misaligned pointer (2-byte aligned only), odd ld, K or N not a multiple of 8 -> generic
    assert s(4096, 4096, 4096, A16 + 2, 4096, A16, 4096, A16, 4096) == 0
    assert s(4096, 4096, 4096, A16, 4100, A16, 4096, A16, 4096) == 0
    assert s(4096, 4096, 4095, A16, 4096, A16, 4096, A16, 4096) == 0
    assert s(4096, 4094, 4096, A16, 4096, A16, 4096, A16, 4096) == 0
    # ragged M is fine for the fast path
    assert s(4095, 3000, 1000, A16, 1000, A16, 3000, A16, 3000) > 0


def test_choice_table_names_product_configs():
    """Every config the generated table names is compiled into the product library, is a
    fast config, and takes the layout of its exact entries; the table covers the headline."""
    cfgs = tg.configs()
    t = parse_choice_table()
    exact, model = t["kF16"]
    assert model and exact
    for cfg, coef in model:
        assert cfgs[cfg]["built"] == 1 and cfgs[cfg]["generic"] == 0
        assert all(v >= 0 for v in coef)
    for (lay, M, N, K, cfg) in exact:
        assert cfgs[cfg]["built"] == 1 and (cfgs[cfg]["layouts"] >> lay) & 1
    assert any(e[:4] == (0, 4096, 4096, 4096) for e in exact)
    f8 = tg.fp8_configs()
    exact8, model8 = t["kFp8"]
    assert model8 and exact8
    for cfg, _ in model8:
        assert f8[cfg]["built"] == 1
    for e in exact8:
        assert e[0] == 0 and f8[e[4]]["built"] == 1
    # the tooling-only rows are listed (same indices in both builds) but not compiled here
    assert any(c["built"] == 0 for c in cfgs) and any(c["built"] == 0 for c in f8)


def test_every_product_config_is_reachable():
    """The product library compiles no config that no call can reach: each compiled fast
    config is the selector's pick for some shape (an exact entry of the table or the cost
    model's argmin on a grid of shapes) or the split-K plan's config; the same for fp8."""
    cfgs = tg.configs()
    exact, _ = parse_choice_table()["kF16"]
    reach = {e[4] for e in exact}
    grid = [(M, N, K) for M in range(256, 16385, 768) for N in range(256, 16385, 768)
            for K in (256, 1024, 4096, 16384)]
    for layout in range(4):
        ta, tb = layout >> 1, layout & 1
        for (M, N, K) in grid:
            reach.add(tg.tgemm_select_config_ex(ta, tb, M, N, K, A=A16, B=A16, C=A16))
            reach.add(tg.tgemm_split_plan(ta, tb, M, N, K, A=A16, B=A16, C=A16)[0])
    built = {i for i, c in enumerate(cfgs) if c["built"] and not c["generic"]}
    assert built <= reach, [cfgs[i]["name"] for i in sorted(built - reach)]
    f8 = tg.fp8_configs()
    exact8, _ = parse_choice_table()["kFp8"]
    reach8 = {e[4] for e in exact8}
    for (M, N, K) in grid:
        reach8.add(tg.tgemm_fp8_select_config(M, N, K, A=A16, B=A16, C=A16))
    built8 = {i for i, c in enumerate(f8) if c["built"] and c["name"].startswith("f")}
    assert built8 <= reach8, [f8[i]["name"] for i in sorted(built8 - reach8)]


SELECT_SHAPES = [(1024, 1024, 1024), (2048, 2048, 4096), (2560, 2560, 4096), (16384, 512, 4096),
                 (3072, 3072, 4096), (4095, 3000, 1000), (3584, 3584, 2048), (4096, 4096, 4096),
                 (6144, 6144, 4096), (5120, 4096, 4096), (8192, 8192, 8192), (1000, 1000, 3000),
                 (7000, 5000, 1536), (12288, 4096, 4096), (640, 20480, 2048), (2304, 2304, 6144)]


@pytest.mark.parametrize("layout", [0, 1, 2, 3])
def test_select_follows_choice_table(layout):
    """tgemm_select_config_ex returns the table's exact entry for a timed shape and the cost
    model's argmin elsewhere (recomputed here from the parsed table)."""
    cfgs = tg.configs()
    exact, model = parse_choice_table()["kF16"]
    ta, tb = layout >> 1, layout & 1
    ok = lambda c: cfgs[c]["built"] and not cfgs[c]["generic"] and (cfgs[c]["layouts"] >> layout) & 1
    tile_of = lambda c: (cfgs[c]["block_m"], cfgs[c]["block_n"])
    shapes = SELECT_SHAPES + [e[1:4] for e in exact if e[0] == layout]
    for (M, N, K) in shapes:
        got = tg.tgemm_select_config_ex(ta, tb, M, N, K, A=A16, B=A16, C=A16)
        # fast configs need 8-element chunks along each operand's contiguous dimension
        eligible = ((M if ta else K) % 8 == 0 and (K if tb else N) % 8 == 0 and N % 8 == 0)
        want = expected_choice(exact, model, layout, M, N, K, tile_of, ok) if eligible else 0
        assert got == want, (layout, M, N, K, got, want)


def test_gemm_rejects_invalid_before_hip():
    # invalid arguments are reported before any HIP call (works with no GPU present)
    assert tg.gemm_f16_raw(-1, 8, 8, A16, 8, A16, 8, A16, 8, 1, None) == tg.TGEMM_EINVAL_DIM
    assert tg.gemm_f16_raw(8, 8, 8, A16, 4, A16, 8, A16, 8, 1, None) == tg.TGEMM_EINVAL_LD
    assert tg.gemm_f16_raw(8, 8, 8, 0, 8, A16, 8, A16, 8, 1, None) == tg.TGEMM_ENULL
    assert tg.gemm_f16_raw(0, 8, 8, 0, 8, 0, 8, 0, 8, 1, None) == tg.TGEMM_OK  # no-op
    assert tg.gemm_f16_cfg_raw(99, 8, 8, 8, A16, 8, A16, 8, A16, 8, 1, None) == tg.TGEMM_EINVAL_CFG
    assert tg.gemm_f16_cfg_raw(1, 8, 8, 8, A16 + 2, 8, A16, 8, A16, 8, 1, None) == tg.TGEMM_EINVAL_CFG


def test_config_layouts():
    """Every config takes A and B as given; the generic kernel and the ping-pong configs
    the selector uses for transposed operands take all four layouts."""
    cfgs = tg.configs()
    for c in cfgs:
        assert c["layouts"] & 1 and c["layouts"] in (1, 0xF)
    assert cfgs[0]["layouts"] == 0xF
    P = dict(A=A16, B=A16, C=A16)
    for ta in (0, 1):
        for tb in (0, 1):
            for M, N, K in [(4096, 4096, 4096), (1024, 1024, 1024), (16384, 512, 4096), (4096, 3000, 1000)]:
                idx = tg.tgemm_select_config_ex(ta, tb, M, N, K, **P)
                assert idx >= 0 and cfgs[idx]["layouts"] & (1 << (2 * ta + tb)), (ta, tb, M, N, K, idx)


def test_select_ex_leading_dimensions_and_eligibility():
    s = tg.tgemm_select_config_ex
    # A^T is K x M: lda >= M; B^T is N x K: ldb >= K
    assert s(1, 0, 64, 64, 128, A16, 63, A16, 64, A16, 64) == tg.TGEMM_EINVAL_LD
    assert s(1, 0, 64, 64, 128, A16, 64, A16, 64, A16, 64) > 0
    assert s(0, 1, 64, 64, 128, A16, 128, A16, 127, A16, 64) == tg.TGEMM_EINVAL_LD
    assert s(0, 1, 64, 64, 128, A16, 128, A16, 128, A16, 64) > 0
    # the contiguous dimension decides the fast path: M for A^T, K for B^T, N for C
    assert s(1, 0, 4092, 4096, 4096, A16, 4096, A16, 4096, A16, 4096) == 0
    assert s(0, 0, 4092, 4096, 4096, A16, 4096, A16, 4096, A16, 4096) > 0
    assert s(1, 0, 4096, 4096, 4092, A16, 4096, A16, 4096, A16, 4096) > 0
    assert s(0, 1, 4096, 4096, 4092, A16, 4096, A16, 4096, A16, 4096) == 0
    assert s(0, 1, 4096, 4092, 4096, A16, 4096, A16, 4096, A16, 4096) == 0
    # the NN form is the (0, 0) case of the ex form
    for M, N, K in [(4096, 4096, 4096), (100, 104, 96), (1024, 1024, 1024)]:
        args = (M, N, K, A16, K, A16, N, A16, N)
        assert tg.tgemm_select_config(*args) == s(0, 0, *args)
    # a config that only takes A and B as given refuses transposed operands
    nn_only = [i for i, c in enumerate(tg.configs()) if c["layouts"] == 1][0]
    assert tg.gemm_f16_ex_cfg_raw(nn_only, 1, 0, 256, 256, 256, A16, 256, A16, 256, A16, 256, 1,
                                  None) == tg.TGEMM_EINVAL_CFG
    assert tg.gemm_f16_ex_raw(1, 0, 8, 8, 8, A16, 7, A16, 8, A16, 8, 1, None) == tg.TGEMM_EINVAL_LD


def test_split_plans_and_workspace_sizes():
    """Shapes without a split entry in the table take the rule: small grids split to about
    one workgroup per compute unit; grids that fill the GPU do not split and need no
    workspace. Every plan, from the table or the rule, stays within one round of workgroups
    with at least 64 k-tiles per split."""
    plan = tg.tgemm_split_plan
    cfgs = tg.configs()
    timed = {e[:4] for e in parse_choice_table()["kSplit"]}
    for ta in (0, 1):
        for tb in (0, 1):
            for (M, N, K), want in [((1024, 1024, 32768), 4), ((512, 512, 16384), 8), ((2048, 2048, 16384), 2),
                                    ((512, 4096, 4096), 2), ((1024, 1024, 1024), 1), ((16384, 512, 4096), 1),
                                    ((4096, 1024, 8192), 1), ((4096, 4096, 4096), 1), ((4095, 3000, 1000), 1),
                                    ((8192, 8192, 8192), 1)]:
                cfg, sp, wb = plan(ta, tb, M, N, K)
                if (2 * ta + tb, M, N, K) not in timed:
                    assert sp == want, (M, N, K, cfg, sp)
                c = cfgs[cfg]
                tiles = -(-M // c["block_m"]) * -(-N // c["block_n"])
                assert wb == (4096 + tiles * sp * c["block_m"] * c["block_n"] * 4 if sp > 1 else 0)
                assert tg.tgemm_workspace_bytes(ta, tb, M, N, K) == wb
                if sp > 1:
                    assert c["layouts"] == 0xF and tiles * sp <= 256
                    assert -(-K // c["block_k"]) // sp >= 64
    # generic arguments never split
    assert plan(0, 0, 1024, 1024, 1020)[1] == 1 and plan(0, 0, 1024, 1024, 1020)[2] == 0


def test_split_plan_follows_table():
    """A shape the table sweep timed split options on takes the table's plan: the unsplit
    choice (cfg -1) or the listed (cfg, splits), which is split-capable and bounded like the
    rule's plans."""
    cfgs = tg.configs()
    entries = parse_choice_table()["kSplit"]
    for (lay, M, N, K, cfg, splits) in entries:
        got = tg.tgemm_split_plan(lay >> 1, lay & 1, M, N, K, A=A16, B=A16, C=A16)
        if cfg < 0:
            assert got[1] == 1 and got[0] == tg.tgemm_select_config_ex(lay >> 1, lay & 1, M, N, K, A=A16, B=A16,
                                                                       C=A16), (lay, M, N, K, got)
        else:
            assert got[:2] == (cfg, splits), (lay, M, N, K, got)
            c = cfgs[cfg]
            assert c["built"] and c["layouts"] == 0xF and 2 <= splits <= 8
            assert -(-M // c["block_m"]) * -(-N // c["block_n"]) * splits <= 256


def test_workspace_errors_before_hip():
    L = tg.lib()
    M, N, K = 1024, 1024, 32768  # a shape that splits
    args = (0, 0, M, N, K, A16, K, A16, N, A16, N, 1)
    need = tg.tgemm_workspace_bytes(0, 0, M, N, K)
    assert L.gemm_f16_ws(*args, None, 0, None) == tg.TGEMM_ENULL
    assert L.gemm_f16_ws(*args, A16 + 16, need, None) == tg.TGEMM_EALIGN
    assert L.gemm_f16_ws(*args, A16, need - 1, None) == tg.TGEMM_EWORKSPACE
    assert L.gemm_f16_ws_cfg(15, 9, *args, A16, need, None) == tg.TGEMM_EINVAL_CFG     # > 8 splits
    assert L.gemm_f16_ws_cfg(7, 2, *args, A16, need, None) == tg.TGEMM_EINVAL_CFG      # not split-capable
    assert L.gemm_f16_ws_cfg(15, 4, *args, A16, need - 1, None) == tg.TGEMM_EWORKSPACE
    assert L.gemm_f16_ws_cfg(15, 4, 0, 0, 64, 64, 64, A16, 64, A16, 64, A16, 64, 1, A16, 1 << 30,
                             None) == tg.TGEMM_EINVAL_CFG                                  # 4 splits of 2 k-tiles
    # (a shape that does not split needs no workspace: covered on the GPU, since such a call
    # goes on to launch)
    assert tg.tgemm_strerror(tg.TGEMM_EWORKSPACE) != "unknown error code"


def test_grouped_validation_before_hip():
    """Every descriptor is checked before anything is enqueued (no GPU needed)."""
    import ctypes
    L = tg.lib()
    good = tg.GemmDesc(256, 256, 256, A16, 256, A16, 256, A16, 256)
    bad_ld = tg.GemmDesc(256, 256, 256, A16, 255, A16, 256, A16, 256)
    bad_null = tg.GemmDesc(256, 256, 256, 0, 256, A16, 256, A16, 256)
    arr = (tg.GemmDesc * 3)(good, bad_ld, good)
    assert L.gemm_f16_grouped(0, 0, 3, arr, 1, None) == tg.TGEMM_EINVAL_LD
    arr = (tg.GemmDesc * 2)(good, bad_null)
    assert L.gemm_f16_grouped(0, 0, 2, arr, 1, None) == tg.TGEMM_ENULL
    assert L.gemm_f16_grouped(0, 0, 1, None, 1, None) == tg.TGEMM_ENULL
    assert L.gemm_f16_grouped(0, 0, -1, None, 1, None) == tg.TGEMM_EINVAL_DIM
    assert L.gemm_f16_grouped(0, 0, 0, None, 1, None) == tg.TGEMM_OK
    # transposed A: lda >= M
    tA = tg.GemmDesc(256, 128, 64, A16, 200, A16, 128, A16, 128)
    assert L.gemm_f16_grouped(1, 0, 1, (tg.GemmDesc * 1)(tA), 1, None) == tg.TGEMM_EINVAL_LD
    assert ctypes.sizeof(tg.GemmDesc) == 72


SHAPES = [(1, 1), (255, 257), (256, 256), (1024, 1024), (4096, 4096), (4095, 3000), (8192, 8192),
          (16384, 512), (3000, 4095), (1000, 64), (64, 1000), (2304, 2304), (513, 129)]


@pytest.mark.parametrize("M,N", SHAPES)
def test_tile_map_is_bijection(M, N):
    for idx in range(tg.tgemm_num_configs()):
        c = tg.tgemm_config_desc(idx)
        tm = -(-M // c["block_m"])
        tn = -(-N // c["block_n"])
        nwg = tg.tgemm_num_workgroups(idx, M, N)
        assert nwg == tm * tn
        if nwg > 70000:
            continue
        seen = set()
        for wg in range(nwg):
            t = tg.tgemm_tile_of(idx, M, N, wg)
            assert 0 <= t[0] < tm and 0 <= t[1] < tn, (idx, wg, t)
            seen.add(t)
        assert len(seen) == nwg, (idx, M, N)
        with pytest.raises(tg.TgemmError):
            tg.tgemm_tile_of(idx, M, N, nwg)


def test_tile_map_keeps_xcd_tiles_together():
    """With the XCD remap, the tiles one XCD runs (hardware ids x, x+8, x+16, ...) form
    a compact block: at 4096^2 with 256^2 tiles each XCD gets a 4 x 8 block."""
    idx = next(i for i, c in enumerate(tg.configs())
               if (c["block_m"], c["block_n"], c["xcd_remap"], c["panel"]) == (256, 256, 1, 4))
    for x in range(8):
        tiles = [tg.tgemm_tile_of(idx, 4096, 4096, wg) for wg in range(x, 256, 8)]
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(tiles) == 32 and len(rows) == 4 and len(cols) == 8, (x, rows, cols)


@pytest.mark.parametrize("M,N,splits", [(1024, 1024, 4), (16384, 512, 2), (4096, 1024, 2), (2048, 2048, 3),
                                          (1000, 520, 8), (256, 256, 5)])
def test_split_tile_map(M, N, splits):
    """The split-K map covers every (tile, split) once, equals tgemm_tile_of at one split,
    and, with XCD-remapped configs, gives each XCD (hardware id % 8) one split only where
    the splits divide the XCDs' equal shares."""
    for idx in range(tg.tgemm_num_configs()):
        c = tg.tgemm_config_desc(idx)
        if c["generic"] or c["layouts"] != 0xF:  # the configs that cannot split
            with pytest.raises(tg.TgemmError):
                tg.tgemm_split_tile_of(idx, M, N, 2, 0)
            continue
        tiles = tg.tgemm_num_workgroups(idx, M, N)
        got = [tg.tgemm_split_tile_of(idx, M, N, splits, wg) for wg in range(tiles * splits)]
        assert len(set(got)) == tiles * splits
        tn = -(-N // c["block_n"])
        assert all(0 <= s < splits and 0 <= a * tn + b < tiles for a, b, s in got)
        assert [t[:2] for t in (tg.tgemm_split_tile_of(idx, M, N, 1, wg) for wg in range(tiles))] == \
            [tg.tgemm_tile_of(idx, M, N, wg) for wg in range(tiles)]
        if c["xcd_remap"] and (tiles * splits) % 8 == 0 and tiles % ((tiles * splits) // 8) == 0:
            for x in range(8):
                assert len({s for wg, (_, _, s) in enumerate(got) if wg % 8 == x}) == 1, (idx, x)
        with pytest.raises(tg.TgemmError):
            tg.tgemm_split_tile_of(idx, M, N, splits, tiles * splits)


def test_tile_maps_refuse_dims_past_the_cap():
    """M or N at TGEMM_MAX_DIM (2^31) is refused by the tile maps as by every entry point,
    so the workgroup counts they compute stay far from int64 overflow."""
    big = 1 << 31
    for idx in range(tg.tgemm_num_configs()):
        assert tg.tgemm_num_workgroups(idx, big, 8) == -1 and tg.tgemm_num_workgroups(idx, 8, big) == -1
        assert tg.tgemm_num_workgroups(idx, big - 1, 8) > 0
        for M, N in ((big, 8), (8, big), (big << 20, big << 20)):
            with pytest.raises(tg.TgemmError):
                tg.tgemm_tile_of(idx, M, N, 0)
            with pytest.raises(tg.TgemmError):
                tg.tgemm_split_tile_of(idx, M, N, 1, 0)


def test_split_tile_map_shares_panels_per_xcd():
    """16384 x 512 on 256^2 tiles in two splits (256 workgroups): each XCD runs one split
    (half of k) of 32 tiles, both tile columns of 16 tile rows, so each A row panel's half
    of k is fetched into one L2."""
    idx = next(i for i, c in enumerate(tg.configs()) if c["name"] == "m256x256x32_s4_w2x4_p4_x1")
    for x in range(8):
        got = [tg.tgemm_split_tile_of(idx, 16384, 512, 2, wg) for wg in range(x, 256, 8)]
        tiles = {(a, b) for a, b, _ in got}
        assert len(got) == 32 and len(tiles) == 32 and len({s for _, _, s in got}) == 1, (x, tiles)
        assert len({a for a, _ in tiles}) == 16 and len({b for _, b in tiles}) == 2, (x, tiles)


# ---------------------------------------------------------------- fp8 block-scaled path
def test_fp8_config_table():
    cfgs = tg.fp8_configs()
    assert len(cfgs) == tg.tgemm_fp8_num_configs() == 5  # test_gpu_fp8.FP8_TABLE_CONFIGS
    for c in cfgs:
        assert c["block_k"] == 128 and c["generic"] == 0 and c["layouts"] == 2
        assert c["block_m"] % 128 == 0 and c["block_n"] % 128 == 0
        waves = c["waves_m"] * c["waves_n"]
        # operand ring + three groups of A row scales (4 k-tiles each) + a spare 256 bytes
        # for copies with nothing to fetch
        ring = c["stages"] * (c["block_m"] + c["block_n"]) * 128
        assert c["lds_bytes"] == ring + 3 * c["block_m"] * 4 * 4 + 256
        assert c["lds_bytes"] <= 160 * 1024
        assert 128 % (c["block_n"] // c["waves_n"]) == 0   # a wave's columns in one scale block
        assert c["block_m"] <= 64 * waves                    # a slice of A scales: one copy per wave
    with pytest.raises(tg.TgemmError):
        tg.tgemm_fp8_config_desc(len(cfgs))


def test_fp8_select():
    s = tg.tgemm_fp8_select_config
    f8 = tg.fp8_configs()
    exact, model = parse_choice_table()["kFp8"]
    ok = lambda c: f8[c]["built"] == 1
    tile_of = lambda c: (f8[c]["block_m"], f8[c]["block_n"])
    for (M, N, K) in SELECT_SHAPES + [e[1:4] for e in exact]:
        if N % 8 or K % 16:
            continue
        assert s(M, N, K) == expected_choice(exact, model, 0, M, N, K, tile_of, ok), (M, N, K)
    assert s(0, 8, 16) == tg.SELECT_NOOP and s(8, 8, 0) == tg.SELECT_ZERO_FILL
    # generic kernel: K or ld not a multiple of 16, N or ldc not a multiple of 8, unaligned
    assert s(256, 256, 100) == tg.FP8_GENERIC
    assert s(256, 256, 256, lda=264) == tg.FP8_GENERIC
    assert s(256, 252, 256) == tg.FP8_GENERIC
    assert s(256, 256, 256, A=256 + 8) == tg.FP8_GENERIC
    assert s(256, 256, 256, C=256 + 2) == tg.FP8_GENERIC
    assert s(255, 256, 4000) >= 0                         # ragged M and K (16 | K) stay fast
    # any ld at or above K is valid: byte strides past 2^23 take the generic kernel
    fast = s(256, 256, 256)
    assert fast >= 0 and s(256, 256, 256, lda=1 << 23) == fast
    assert s(256, 256, 256, lda=(1 << 23) + 16) == tg.FP8_GENERIC
    assert s(256, 256, 256, ldb=(1 << 23) + 16) == tg.FP8_GENERIC
    assert s(256, 256, 256, ldc=(1 << 40)) == fast
    # errors
    assert s(-1, 8, 8) == tg.TGEMM_EINVAL_DIM
    assert s(8, 8, 32, lda=16) == tg.TGEMM_EINVAL_LD
    assert s(8, 8, 32, ldb=16) == tg.TGEMM_EINVAL_LD
    assert s(8, 8, 32, ldc=4) == tg.TGEMM_EINVAL_LD
    assert s(8, 8, 32, A=0) == tg.TGEMM_ENULL
    assert s(8, 8, 32, C=257) == tg.TGEMM_EALIGN


def test_fp8_gemm_rejects_invalid_before_hip():
    g = tg.gemm_fp8_block_raw
    P, S = 256, 512   # aligned fake pointers (never dereferenced: every call returns early)
    assert g(-1, 8, 16, P, 16, S, P, 16, S, P, 8, 0, None) == tg.TGEMM_EINVAL_DIM
    assert g(8, 8, 16, P, 8, S, P, 16, S, P, 8, 0, None) == tg.TGEMM_EINVAL_LD
    assert g(8, 8, 16, P, 16, 0, P, 16, S, P, 8, 0, None) == tg.TGEMM_ENULL     # scale_a
    assert g(8, 8, 16, P, 16, S, P, 16, 0, P, 8, 0, None) == tg.TGEMM_ENULL     # scale_b
    assert g(8, 8, 16, P, 16, S + 2, P, 16, S, P, 8, 0, None) == tg.TGEMM_EALIGN
    assert g(0, 8, 16, 0, 16, 0, 0, 16, 0, 0, 8, 0, None) == tg.TGEMM_OK          # no-op
    c = tg.gemm_fp8_block_cfg_raw
    assert c(7, 8, 8, 16, P, 16, S, P, 16, S, P, 8, 0, None) == tg.TGEMM_EINVAL_CFG
    assert c(-1, 8, 8, 16, P, 16, S, P, 16, S, P, 8, 0, None) == tg.TGEMM_EINVAL_CFG
    # a fast config cannot take K = 100: rejected, not silently run
    assert c(0, 8, 8, 100, P, 100, S, P, 100, S, P, 8, 0, None) == tg.TGEMM_EINVAL_CFG


def test_fp8_quant_rejects_invalid_before_hip():
    q = tg.quant_fp8_block_raw
    P, S = 256, 512
    assert q(8, 128, P, 128, 2, P, 128, S, None) == tg.TGEMM_EINVAL_DIM       # block_rows
    assert q(-1, 128, P, 128, 1, P, 128, S, None) == tg.TGEMM_EINVAL_DIM
    assert q(8, 128, P, 64, 1, P, 128, S, None) == tg.TGEMM_EINVAL_LD
    assert q(8, 128, P, 128, 1, P, 100, S, None) == tg.TGEMM_EINVAL_LD
    assert q(8, 128, P, 128, 1, P, 128, 0, None) == tg.TGEMM_ENULL
    assert q(8, 128, P + 1, 128, 1, P, 128, S, None) == tg.TGEMM_EALIGN
    assert q(8, 128, P, 128, 128, P, 128, S + 2, None) == tg.TGEMM_EALIGN
    assert q(0, 128, 0, 128, 1, 0, 128, 0, None) == tg.TGEMM_OK               # no-op
    # no upper bound on the strides (the quantizer indexes in 64 bits): a huge ld is not an
    # argument error, so the call goes on to the device check (no GPU here: TGEMM_EDEVICE)
    assert q(8, 128, P, 1 << 40, 1, P, 1 << 40, S, None) in (tg.TGEMM_OK, tg.TGEMM_EDEVICE)


def test_workspace_bytes_cfg():
    """The per-config workspace query is the layout gemm_f16_ws_cfg checks against: 0 when
    unsplit, else 4 KiB of counters plus splits fp32 partial tiles per output tile."""
    q = tg.tgemm_workspace_bytes_cfg
    for idx, c in enumerate(tg.configs()):
        for M, N in ((1, 1), (520, 392), (1024, 1024)):
            assert q(idx, 1, M, N) == 0
            tiles = -(-M // c["block_m"]) * -(-N // c["block_n"])
            splittable = not c["generic"] and c["layouts"] == 0xF and tiles <= 1024
            for splits in (2, 8):
                if splittable:
                    assert q(idx, splits, M, N) == 4096 + tiles * splits * c["block_m"] * c["block_n"] * 4
                else:
                    with pytest.raises(tg.TgemmError):
                        q(idx, splits, M, N)
    with pytest.raises(tg.TgemmError):
        q(tg.tgemm_num_configs(), 1, 8, 8)
    with pytest.raises(tg.TgemmError):
        q(0, 9, 8, 8)
    with pytest.raises(tg.TgemmError):
        q(0, 1, -1, 8)
    # every split plan the library makes fits the static scratch of gemm_f16_ws_static
    for M, N, K in ((512, 512, 16384), (2048, 2048, 131072), (128, 128, 1 << 20), (1024, 1024, 32768)):
        assert tg.tgemm_split_plan(0, 0, M, N, K)[2] <= tg.STATIC_SCRATCH_BYTES


def test_static_entry_rejects_before_hip():
    s = tg.gemm_f16_ws_static_raw
    assert s(0, 0, -1, 8, 8, 256, 8, 256, 8, 256, 8, 0, None) == tg.TGEMM_EINVAL_DIM
    assert s(0, 0, 8, 8, 8, 256, 7, 256, 8, 256, 8, 0, None) == tg.TGEMM_EINVAL_LD
    assert s(0, 0, 8, 8, 8, 0, 8, 256, 8, 256, 8, 0, None) == tg.TGEMM_ENULL
    assert s(0, 0, 0, 8, 8, 0, 8, 0, 8, 0, 8, 0, None) == tg.TGEMM_OK


def test_product_kernels_use_no_scratch():
    """The product build records every kernel's resources (kernel_resources.txt, from the
    compiler's resource remarks) and refuses kernels that use scratch memory or spill: a
    register array moved to scratch puts memory loads and full waits into the copy stream."""
    from tiled_dense_gemm_04_amd import build as B
    if not os.path.exists(B.RESOURCES):
        pytest.skip("library built before the resource report existed")
    text = open(B.RESOURCES).read()
    rows = [ln for ln in text.splitlines() if ln.strip()]
    assert any("gemm_pingpong" in r for r in rows) and any("gemm_fp8_block_kernel" in r for r in rows)
    for r in rows:
        assert "ScratchSize [bytes/lane]=0 " in r and "VGPRs Spill=0" in r and "SGPRs Spill=0" in r, r
    # the parser itself, on a made-up remark pair
    res = B.kernel_resources("x.hip:1:1: remark: Function Name: k [-Rpass-analysis=kernel-resource-usage]\n"
                             "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 20 [-Rpass-analysis=kernel-resource-usage]\n")
    assert B.check_resources(res) == ["k"]


def test_choice_table_is_generated_from_committed_timings():
    """The selector's table (csrc/tgemm_choice.inc) and its report (profiles/config_choice.md)
    are exactly what `sweep.py --refit` makes of the committed sweep timings
    (profiles/config_choice_timings.json) for the configs this build compiles: no hand
    edits, and a config demoted to the tooling build drops out of both."""
    import json
    from tiled_dense_gemm_04_amd import sweep
    with open(os.path.join(ROOT, "profiles", "config_choice_timings.json")) as f:
        data = json.load(f)
    inc, md = sweep.render_table(sweep.product_only(data))
    with open(os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc", "tgemm_choice.inc")) as f:
        assert f.read() == inc
    with open(os.path.join(ROOT, "profiles", "config_choice.md")) as f:
        assert f.read() == md
