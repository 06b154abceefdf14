"""Mutation check of the oracle's pins: plant one plausible mistake at a time
in a copy of oracle.c (a transposed or mis-strided operand, a dropped term, a
wrong sign, an off-by-one loop, a wrong binary16 bias or rounding rule), build
it on the CPU, and require the pin suite to fail against it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrence to replace: 1-based, 0 = all)
MUTANTS = [
    ("B_row_stride_N", "const float *Bk = B + (size_t)k * (size_t)ldb;",
     "const float *Bk = B + (size_t)k * (size_t)N;", 1),
    ("A_row_stride_K", "row_f32(N, K, A + (size_t)i * (size_t)lda, B, ldb, s, g);",
     "row_f32(N, K, A + (size_t)i * (size_t)K, B, ldb, s, g);", 1),
    ("B_transposed_elems", "double b = (double)B[(size_t)k * (size_t)ldb + j];",
     "double b = (double)B[j * (size_t)ldb + (size_t)k];", 1),
    ("beta_term_dropped", "r += beta * (double)C[(size_t)i * (size_t)ldc + j];", "r += 0.0;", 1),
    ("alpha_sign", "double r = use_ab ? alpha * s[j] : 0.0;", "double r = use_ab ? -alpha * s[j] : 0.0;", 1),
    ("alpha_ignored", "double r = use_ab ? alpha * s[j] : 0.0;", "double r = use_ab ? s[j] : 0.0;", 1),
    ("k_starts_at_1", "for (int k = 0; k < K; ++k) {\n        double a = (double)Arow[k];",
     "for (int k = 1; k < K; ++k) {\n        double a = (double)Arow[k];", 1),
    ("k_stops_early", "for (int k = 0; k < K; ++k) {\n        double a = (double)Arow[k];",
     "for (int k = 0; k < K - 1; ++k) {\n        double a = (double)Arow[k];", 1),
    ("G_without_abs", "g[j] += aa * fabs(b);", "g[j] += a * b;", 1),
    ("beta_zero_reads_C", "if (beta != 0.0)\n                        r += beta * (double)C",
     "if (1)\n                        r += beta * (double)C", 1),
    ("alpha_zero_reads_AB", "int use_ab = (alpha != 0.0) && (K > 0);", "int use_ab = (K > 0);", 1),
    ("f16_beta_dropped", "r += beta * oracle_half_to_double(C[(size_t)i * (size_t)ldc + j]);", "r += 0.0;", 1),
    ("f16_exponent_bias", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);", 1),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 1),
    ("f16_ties_away", "(rem == 0.5 && fmod(fl, 2.0) != 0.0)", "(rem == 0.5)", 1),
    ("f16_truncate", "if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))", "if (0)", 1),
    ("f16_no_overflow_check", "if (v > 65504.0)", "if (v > 65504.0 && 0)", 1),
    ("f16_elems_A_stride", "double a = oracle_half_to_double(A[i * (size_t)lda + k]);",
     "double a = oracle_half_to_double(A[i * (size_t)K + k]);", 1),
    ("mixed_beta_dropped", "r += beta * (double)C[(size_t)i * (size_t)ldc + j];", "r += 0.0;", 2),
    ("mixed_C_as_half", "r += beta * (double)C[(size_t)i * (size_t)ldc + j];",
     "r += beta * oracle_half_to_double(((const uint16_t *)C)[(size_t)i * (size_t)ldc + j]);", 2),
    ("mixed_C_rounded_to_half", "r += beta * (double)C[(size_t)i * (size_t)ldc + j];",
     "r += beta * oracle_half_to_double(oracle_double_to_half((double)C[(size_t)i * (size_t)ldc + j]));", 2),
    ("mixed_elems_beta_sign", "r += beta * (double)C[i * (size_t)ldc + j];",
     "r -= beta * (double)C[i * (size_t)ldc + j];", 2),
]


def _mutate(text, old, new, occ):
    assert old in text, old
    if occ == 0:
        return text.replace(old, new)
    idx = -1
    for _ in range(occ):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, occ):
    text = open(SRC).read()
    src = tmp_path / "mutant.c"
    src.write_text(_mutate(text, old, new, occ))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), str(src)], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not ragged and not match_full",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "mutant %s survived the pins:\n%s" % (name, r.stdout[-2000:])


def test_unmutated_copy_passes(tmp_path):
    """Control: the same procedure on an unmodified copy passes."""
    lib = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), SRC], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not ragged and not match_full",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:]
