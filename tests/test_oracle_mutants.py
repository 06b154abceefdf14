"""Mutation check of the oracle's pins: plant one plausible mistake at a time
in a copy of the oracle and require the pin suite to fail against it.

  * oracle.c (a transposed or mis-strided operand, a dropped term, a wrong
    sign, an off-by-one loop, a wrong binary16 bias or rounding rule): the
    copy is built on the CPU and loaded in place of liboracle.so;
  * the Python side, oracle/__init__.py (the acceptance bound, the
    element-wise comparison, the whole-matrix checksum and Freivalds' check):
    the copy is imported as the `oracle` package before the pins run."""
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
    ("f16_decode_ignores_ld", "X[(size_t)r * (size_t)ld + c]", "X[(size_t)r * (size_t)cols + c]", 1),
    ("f16_decoded_B_stride", "const double *Bk = B + (size_t)k * (size_t)N;",
     "const double *Bk = B + (size_t)k * (size_t)K;", 1),
    ("f16_A_row_not_decoded_per_row", "adec[k] = oracle_half_to_double(Arow[k]);",
     "adec[k] = oracle_half_to_double(Arow[0]);", 1),
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


# Mistakes planted in oracle/__init__.py: (name, text, replacement, occurrence).
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = [
    # tolerance(): the bound every parity test accepts against
    ("tol_f32_uses_f16_unit", "u_out, eta = U32, ETA32", "u_out, eta = U16, ETA32", 1),
    ("tol_f16_uses_f32_unit", "u_out, eta = U16, ETA16", "u_out, eta = U32, ETA16", 1),
    ("tol_f16_eta_of_f32", "u_out, eta = U16, ETA16", "u_out, eta = U16, ETA32", 1),
    ("tol_beta_C_dropped", "mag = abs(float(alpha)) * G + abs(float(beta)) * Cabs",
     "mag = abs(float(alpha)) * G", 1),
    ("tol_alpha_not_abs", "mag = abs(float(alpha)) * G", "mag = float(alpha) * G", 1),
    ("tol_factor_4_to_1", "4.0 * max(int(K), 1)", "1.0 * max(int(K), 1)", 1),
    ("tol_K_not_max1", "4.0 * max(int(K), 1)", "4.0 * int(K)", 1),
    ("tol_no_out_rounding_factor", "(1.0 + u_out) * 4.0", "4.0", 1),
    ("tol_no_R_term", "+ u_out * np.abs(R) + eta", "+ eta", 1),
    ("tol_no_eta", "+ u_out * np.abs(R) + eta", "+ u_out * np.abs(R)", 1),
    # compare(): the element-wise verdict
    ("cmp_strict_less", "return bool(worst <= 1.0)", "return bool(worst < 1.0)", 1),
    ("cmp_nan_only_R", "both_nan = np.isnan(g) & np.isnan(R)", "both_nan = np.isnan(R)", 1),
    ("cmp_nan_only_gpu", "both_nan = np.isnan(g) & np.isnan(R)", "both_nan = np.isnan(g)", 1),
    ("cmp_signed_error", "err = np.abs(g - R)", "err = g - R", 1),
    ("cmp_any_inf_passes", "ratio = np.where(inf_r & (g == R), 0.0, ratio)",
     "ratio = np.where(inf_r, 0.0, ratio)", 1),
    # checksum(): the whole-matrix sum and its magnitude
    ("sum_beta_mag_dropped", "mag += abs(float(beta)) * float(np.abs(C2).sum())", "mag += 0.0", 1),
    ("sum_alpha_mag_signed", "np.abs(A2).sum(axis=0) @ np.abs(B2).sum(axis=1)",
     "A2.sum(axis=0) @ np.abs(B2).sum(axis=1)", 1),
    ("sum_beta_term_sign", "exp += float(beta) * float(C2.sum())",
     "exp -= float(beta) * float(C2.sum())", 1),
    ("sum_B_colsum", "rb = B2.sum(axis=1)", "rb = B2.sum(axis=0)[:B2.shape[0]]", 1),
    # freivalds(): the product check
    ("frv_beta_mag_dropped", "mag += abs(float(beta)) * (np.abs(C2) @ np.abs(x))", "mag += 0.0", 1),
    ("frv_x_not_abs", "(np.abs(B2) @ np.abs(x))", "(np.abs(B2) @ x)", 1),
    ("frv_beta_dropped", "y += float(beta) * (C2 @ x)", "y += 0.0", 1),
    ("frv_B_transposed", "y += float(alpha) * (A2 @ (B2 @ x))",
     "y += float(alpha) * (A2 @ (B2.T[:B2.shape[0]] @ x[:B2.shape[0]]))", 1),
    # _view2(): the padded-buffer view used by both whole-matrix checks
    ("view_ignores_ld", "strides=(ld * a.itemsize, a.itemsize)",
     "strides=(cols * a.itemsize, a.itemsize)", 1),
]

_RUN_WITH_PACKAGE = (
    "import sys; sys.path.insert(0, sys.argv[1]); import oracle; "
    "assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__; "
    "import pytest; sys.exit(pytest.main(sys.argv[2:]))")


def _run_pins_with_package(pkg_root):
    from oracle.build import LIB, build_oracle
    if not os.path.exists(LIB):
        build_oracle()
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=LIB, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-c", _RUN_WITH_PACKAGE, str(pkg_root), "-x", "-q",
                           "-p", "no:cacheprovider", "-k", "not ragged and not match_full",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def _package_copy(tmp_path, text):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(text)
    for name in ("build.py", "oracle.c"):
        (pkg / name).write_text(open(os.path.join(ROOT, "oracle", name)).read())
    return tmp_path


@pytest.mark.parametrize("name,old,new,occ", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_planted_python_mistake(tmp_path, name, old, new, occ):
    text = open(PY_SRC).read()
    r = _run_pins_with_package(_package_copy(tmp_path, _mutate(text, old, new, occ)))
    assert r.returncode != 0, "mutant %s survived the pins:\n%s" % (name, r.stdout[-2000:])


def test_unmutated_python_copy_passes(tmp_path):
    """Control: the same procedure on an unmodified copy of the package passes."""
    r = _run_pins_with_package(_package_copy(tmp_path, open(PY_SRC).read()))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
