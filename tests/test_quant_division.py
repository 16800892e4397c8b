"""The block quantizer divides by the block scale with one reciprocal per block and a
corrected product per element (tgemm_fp8.hip, div_by_scale), and forms the scale amax / 448
itself as a corrected product (block_scale). quant_division_check.c replays both sequences
on the CPU for every binary16 block maximum and every binary16 x with |x| <= amax (about
10^9 pairs) and checks them against IEEE float32 division bit for bit. No GPU."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_division_is_exact(tmp_path):
    exe = str(tmp_path / "qdc")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quant_division_check.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
