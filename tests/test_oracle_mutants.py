"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a dropped term, a
wrong sign, index or constant, a transposed operand), builds it, and runs the
pin suites (test_oracle_pack.py, test_oracle_attention.py) against that build
in a subprocess. Every mutant must make at least one pin fail.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "bao_ref.c")

MUTANTS = {
    "sigma_drops_factor_2": ("return d - 2 * h;", "return d - h;"),
    "sign_of_zero_negative": ("if (v < 0.0f) bits", "if (v <= 0.0f) bits"),
    "mu_over_padded_width": ("*mu = (float)(asum / d);", "*mu = (float)(asum / (32 * W));"),
    "no_temperature": ("const double inv_sqrt_d = 1.0 / sqrt((double)d);", "const double inv_sqrt_d = 1.0 / d;"),
    "bias_subtracted": ("(double)sg * inv_sqrt_d +", "(double)sg * inv_sqrt_d -"),
    "relpos_rows_swapped": ("(ri - rj + gh - 1)", "(rj - ri + gh - 1)"),
    "dense_bias_transposed": ("((int64_t)h * N + i) * N + j;", "((int64_t)h * N + j) * N + i;"),
    "softmax_wrong_max": ("pt[j] = exp(s[j] - m);", "pt[j] = exp(s[j] - s[0]);"),
    "p8_scale_256": ("double x = rint(255.0 * pt[j]);", "double x = rint(256.0 * pt[j]);"),
    "p8_truncates": ("double x = rint(255.0 * pt[j]);", "double x = floor(255.0 * pt[j]);"),
    "v_scale_128": ("const float inv = 127.0f / amax;", "const float inv = 128.0f / amax;"),
    "v_rounds_toward_zero": ("float r = rintf(decode1(v, dtype, base + (int64_t)j * d + c) * inv);",
                             "float r = truncf(decode1(v, dtype, base + (int64_t)j * d + c) * inv);"),
    "dequant_256": (": 255.0 * l;", ": 256.0 * l;"),
    "norm_p8_off_by_one": ("? (double)psum :", "? (double)psum + 1.0 :"),
    "norm_p8_is_float_sum": ("? (double)psum :", "? 255.0 * l :"),
    "pv_channel_reversed": ("A[c] += pj * vj[c];", "A[c] += pj * vj[d - 1 - c];"),
    "l_from_squares": ("pt[j] = exp(s[j] - m); l += pt[j];", "pt[j] = exp(s[j] - m); l += pt[j] * pt[j];"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "round16_floor": ("double r = rint(a / quantum) * quantum;", "double r = floor(a / quantum) * quantum;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = tmp_path / "bao_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libbao_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                    "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, BAO_REF_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pack.py"),
                        os.path.join(HERE, "test_oracle_attention.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
