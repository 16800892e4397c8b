"""Planted mistakes in copies of the oracle's C source must each fail a pin.

Every mutant below is one plausible slip (a dropped term, a wrong sign, a transposed
index, an off-by-one exponent, a missing or inverted ReLU, a wrong rounding). Each is
compiled from a temporary copy of tgemm_ref.c and the whole pin list runs against it
in a child process (a transposed index may read out of bounds, so a crash counts as
caught). The real oracle is never modified. CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (name, original text, replacement) -- each original must occur exactly once.
MUTANTS = [
    ("dropped_last_term", "for (int64_t k = 0; k < K; ++k) {\n            double a",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            double a"),
    ("dropped_first_term", "for (int64_t k = 0; k < K; ++k) {\n            double a",
     "for (int64_t k = 1; k < K; ++k) {\n            double a"),
    ("entries_dropped_term", "for (int64_t k = 0; k < K; ++k)\n            acc +=",
     "for (int64_t k = 0; k + 1 < K; ++k)\n            acc +="),
    ("subtract_instead_of_add", "acc[j] += a * brow[j];", "acc[j] -= a * brow[j];"),
    ("transposed_A_index", "double a = oracle_f16_decode(A[i * lda + k]);",
     "double a = oracle_f16_decode(A[k * lda + i]);"),
    ("transposed_B_index", "Bd[k * N + j] = oracle_f16_decode(B[k * ldb + j]);",
     "Bd[k * N + j] = oracle_f16_decode(B[j * ldb + k]);"),
    ("ignores_lda", "double a = oracle_f16_decode(A[i * lda + k]);",
     "double a = oracle_f16_decode(A[i * K + k]);"),
    ("entries_swapped_row_col", "oracle_f16_decode(A[rows[t] * lda + k])",
     "oracle_f16_decode(A[cols[t] * lda + k])"),
    ("exponent_bias_off_by_one", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("subnormal_scale_wrong", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("sign_bit_ignored", "return s ? -v : v;", "return v;"),
    ("relu_missing", "acc[j] = relu_d(acc[j]);", "acc[j] = acc[j];"),
    ("relu_inverted", "return x > 0.0 ? x : 0.0;", "return x < 0.0 ? x : 0.0;"),
    ("relu_keeps_negatives_small", "return x > 0.0 ? x : 0.0;", "return x > -1e-3 ? x : 0.0;"),
    ("encode_truncates", "double r = nearbyint(n);", "double r = floor(n);"),
    ("encode_ties_away", "double r = nearbyint(n);", "double r = round(n);"),
    ("encode_overflow_early", "if (a >= 65520.0) return sign | 0x7C00;",
     "if (a > 65504.0) return sign | 0x7C00;"),
    ("encode_subnormal_floor", "if (ex < -14) ex = -14;", "if (ex < -15) ex = -15;"),
]

# The same for the fp8 oracle (tgemm_fp8_ref.c), run against the fp8 pins.
FP8_MUTANTS = [
    ("e4m3_bias_off_by_one", "ldexp((double)(8 + f), e - 10)", "ldexp((double)(8 + f), e - 9)"),
    ("e4m3_subnormal_scale", "v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),
    ("e4m3_nan_whole_top_binade", "if (e == 15 && f == 7)", "if (e == 15)"),
    ("e4m3_encode_truncates", "int64_t q = (int64_t)nearbyint(n);", "int64_t q = (int64_t)floor(n);"),
    ("e4m3_encode_ties_away", "int64_t q = (int64_t)nearbyint(n);", "int64_t q = (int64_t)round(n);"),
    ("e4m3_saturates_early", "if (a >= 448.0) return sign | 0x7E;", "if (a > 400.0) return sign | 0x7E;"),
    ("e4m3_subnormal_floor", "if (ex < -6) ex = -6;", "if (ex < -7) ex = -7;"),
    ("block_of_64", "#define FP8_BLOCK 128", "#define FP8_BLOCK 64"),
    ("a_scale_ignored", "acc += ((double)sarow[kb] * (double)sbrow[kb]) * p;", "acc += (double)sbrow[kb] * p;"),
    ("first_a_scale_only", "acc += ((double)sarow[kb] * (double)sbrow[kb]) * p;",
     "acc += ((double)sarow[0] * (double)sbrow[kb]) * p;"),
    ("b_scale_row_fixed", "SB + (j / FP8_BLOCK) * KB);\n            C[i * ldc + j]", "SB);\n            C[i * ldc + j]"),
    ("last_block_dropped", "for (int64_t kb = 0; kb < KB; ++kb) {\n        const int64_t k0",
     "for (int64_t kb = 0; kb + 1 < KB; ++kb) {\n        const int64_t k0"),
    ("block_tail_dropped", "double p = 0.0; /* exact */\n        for (int64_t k = k0; k < k1; ++k)",
     "double p = 0.0; /* exact */\n        for (int64_t k = k0; k + 1 < k1; ++k)"),
    ("b_operand_transposed", "oracle_e4m3_decode(arow[k]) * oracle_e4m3_decode(wrow[k])",
     "oracle_e4m3_decode(arow[k]) * oracle_e4m3_decode(wrow[k % 8])"),
    ("fp8_relu_missing", "C[i * ldc + j] = relu ? relu_d(v) : v;", "C[i * ldc + j] = v;"),
    ("quant_amax_first_row", "for (int64_t r = r0; r < r1; ++r)\n                for (int64_t k = k0; k < k1; ++k) {\n"
     "                    const float v", "for (int64_t r = r0; r < r0 + 1; ++r)\n                for (int64_t k = k0; "
     "k < k1; ++k) {\n                    const float v"),
    ("quant_divisor_447", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 447.0f : 1.0f"),
    ("quant_zero_block_scale_0", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 448.0f : 0.0f"),
    ("quant_multiplies", "const float y = (float)oracle_f16_decode(X[r * ldx + k]) / s;",
     "const float y = (float)oracle_f16_decode(X[r * ldx + k]) * s;"),
    ("bound_signed_a", "m = fmax(m, fabs(oracle_e4m3_decode(A[i * lda + k])));",
     "m = fmax(m, oracle_e4m3_decode(A[i * lda + k]));"),
]

RUNNER = r"""
import sys, traceback
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from {module} import {pins} as PINS
orc = oracle.Oracle({lib!r})
failed = []
for pin in PINS:
    try:
        pin(orc)
    except Exception:
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
sys.exit(1 if failed else 0)
"""


def _mutant_source(orig, new):
    src = open(oracle.SOURCE).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/present: {orig!r}"
    return src.replace(orig, new)


@pytest.mark.parametrize("name,orig,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, new):
    src = tmp_path / "mut.c"
    src.write_text(_mutant_source(orig, new))
    lib = str(tmp_path / "libmut.so")
    oracle.build(str(src), lib)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib, module="oracle_pins", pins="ALL_PINS")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"


@pytest.mark.parametrize("name,orig,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_mutant_is_caught(tmp_path, name, orig, new):
    src = open(oracle.FP8_SOURCE).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/present: {orig!r}"
    p = tmp_path / "mut_fp8.c"
    p.write_text(src.replace(orig, new))
    lib = str(tmp_path / "libmut.so")
    oracle.build(oracle.SOURCE, lib, fp8_src=str(p))
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib, module="oracle_fp8_pins", pins="FP8_PINS")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"


def test_float_accumulation_is_caught(tmp_path):
    """Accumulating in float32 instead of float64 (rounding every partial sum)."""
    src = open(oracle.SOURCE).read()
    orig = "acc[j] += a * brow[j];"
    assert src.count(orig) == 1
    src = src.replace(orig, "acc[j] = (double)(float)(acc[j] + a * brow[j]);")
    p = tmp_path / "mut.c"
    p.write_text(src)
    lib = str(tmp_path / "libmut.so")
    oracle.build(str(p), lib)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib, module="oracle_pins", pins="ALL_PINS")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, r.stdout
