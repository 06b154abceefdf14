"""Pins for the CPU oracle: each test checks it against something other than
itself -- closed forms, exact rational arithmetic, special matrices whose
product is known, numpy's float64 matmul (BLAS dgemm) and numpy's IEEE
binary16 conversion -- so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them (the mutation
tests in test_oracle_mutants.py check exactly that)."""
from fractions import Fraction
import itertools
import os

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = []

EPS53 = 2.0 ** -53


def _buf(mat, ld, fill=np.nan):
    return wl.pad(np.asarray(mat), ld, fill)


def _exact(M, N, K, alpha, A, B, beta, C):
    """Exact rational value of alpha*A*B + beta*C and of |A||B|."""
    R = [[None] * N for _ in range(M)]
    G = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            g = Fraction(0)
            if alpha != 0:
                for k in range(K):
                    a = Fraction(float(A[i][k]))
                    b = Fraction(float(B[k][j]))
                    s += a * b
                    g += abs(a) * abs(b)
            r = Fraction(alpha) * s
            if beta != 0:
                r += Fraction(beta) * Fraction(float(C[i][j]))
            R[i][j] = r
            G[i][j] = g
    return R, G


# ---------------------------------------------------------------- brute force

_NP = {"f32": np.float32, "f16": np.float16}


@pytest.mark.parametrize("dtype", ["f32", "f16", "f16f32"])
def test_exact_rational_dyadic_all_small_shapes(dtype):
    """Small dyadic inputs (multiples of 1/8 in [-2, 2]): every product and
    partial sum is exact in double, so the oracle must equal the rational
    value exactly, for every M, N, K in 0..4 and several alpha/beta."""
    tin, tc = (_NP[x] for x in wl.operand_types(dtype))
    rng = np.random.default_rng(7)
    for M, N, K in itertools.product(range(0, 5), repeat=3):
        for alpha, beta in [(1.0, 0.0), (-1.5, 0.5), (0.25, -2.0), (0.0, 1.0), (2.0, 1.0)]:
            A = (rng.integers(-16, 17, size=(M, K)) / 8.0).astype(tin)
            B = (rng.integers(-16, 17, size=(K, N)) / 8.0).astype(tin)
            # C carries a 1/4096 part in the mixed case: exact in fp32, not in
            # fp16, so C read through the wrong type cannot pass.
            cfine = (rng.integers(-8, 9, size=(M, N)) / 4096.0) if dtype == "f16f32" else 0.0
            C = (rng.integers(-16, 17, size=(M, N)) / 8.0 + cfine).astype(tc)
            lda, ldb, ldc = K + 1, N + 2, N + 3
            R, G = oracle.gemm(M, N, K, alpha, _buf(A, lda), lda, _buf(B, ldb), ldb,
                               beta, _buf(C, ldc, 7.0), ldc, dtype)
            ER, EG = _exact(M, N, K, alpha, A, B, beta, C)
            for i in range(M):
                for j in range(N):
                    assert Fraction(R[i, j]) == ER[i][j], (M, N, K, alpha, beta, i, j)
                    assert Fraction(G[i, j]) == EG[i][j]


def test_exact_rational_random_f32_within_double_rounding():
    """Random fp32 inputs: the oracle is within (K+3)*2^-53*(|alpha|G+|beta||C|)
    of the exact rational value (products are exact; each addition and the
    alpha/beta steps round once in double)."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        M, N, K = rng.integers(1, 7, size=3)
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = float(np.float32(rng.uniform(-2, 2)))
        A = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
        C = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
        R, G = oracle.gemm(M, N, K, alpha, _buf(A, K), K, _buf(B, N), N, beta, _buf(C, N), N)
        ER, EG = _exact(M, N, K, alpha, A, B, beta, C)
        for i in range(M):
            for j in range(N):
                bound = (K + 3) * EPS53 * (abs(alpha) * float(EG[i][j]) + abs(beta) * abs(float(C[i, j])))
                assert abs(Fraction(R[i, j]) - ER[i][j]) <= Fraction(bound) * Fraction(101, 100)
                assert abs(Fraction(G[i, j]) - EG[i][j]) <= Fraction(K * EPS53 * float(EG[i][j]))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (17, 9, 64), (1, 1, 1000), (64, 33, 257)])
def test_closed_forms(M, N, K):
    alpha, beta = 1.5, -0.5
    C = np.arange(M * N, dtype=np.float32).reshape(M, N) / 4
    # all-ones: R = alpha*K + beta*C, G = K
    A = np.ones((M, K), np.float32)
    B = np.ones((K, N), np.float32)
    R, G = oracle.gemm(M, N, K, alpha, _buf(A, K), K, _buf(B, N), N, beta, _buf(C, N), N)
    np.testing.assert_array_equal(R, alpha * K + beta * C.astype(np.float64))
    np.testing.assert_array_equal(G, np.full((M, N), float(K)))
    # A_ik = 1, B_kj = k: sum_k k = K(K-1)/2
    Bk = np.repeat(np.arange(K, dtype=np.float32)[:, None], N, axis=1)
    R, _ = oracle.gemm(M, N, K, alpha, _buf(A, K), K, _buf(Bk, N), N, 0.0, None, N)
    np.testing.assert_array_equal(R, np.full((M, N), alpha * K * (K - 1) / 2))
    # A_ik = k, B_kj = k: sum_k k^2 = (K-1)K(2K-1)/6
    Ak = np.repeat(np.arange(K, dtype=np.float32)[None, :], M, axis=0)
    R, _ = oracle.gemm(M, N, K, -1.0, _buf(Ak, K), K, _buf(Bk, N), N, 0.0, None, N)
    np.testing.assert_array_equal(R, np.full((M, N), -(K - 1) * K * (2 * K - 1) / 6.0))
    # A_ik = i + 1 (row scale), B_kj = j - 2 (signed column): R_ij = K (i+1)(j-2)
    Ai = np.repeat(np.arange(1, M + 1, dtype=np.float32)[:, None], K, axis=1)
    Bj = np.repeat(np.arange(N, dtype=np.float32)[None, :] - 2, K, axis=0)
    R, G = oracle.gemm(M, N, K, 1.0, _buf(Ai, K + 3), K + 3, _buf(Bj, N + 1), N + 1, 0.0, None, N)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    np.testing.assert_array_equal(R, K * (ii + 1.0) * (jj - 2.0))
    np.testing.assert_array_equal(G, K * (ii + 1.0) * np.abs(jj - 2.0))


def test_identity_and_permutation():
    rng = np.random.default_rng(3)
    M, N = 37, 29
    B = rng.standard_normal((M, N)).astype(np.float32)
    C = rng.standard_normal((M, N)).astype(np.float32)
    eye = np.eye(M, dtype=np.float32)
    # A = I: R = alpha*B + beta*C (each sum has a single nonzero term)
    R, _ = oracle.gemm(M, N, M, 2.0, _buf(eye, M + 1), M + 1, _buf(B, N + 1), N + 1, 0.5, _buf(C, N), N)
    np.testing.assert_array_equal(R, 2.0 * B.astype(np.float64) + 0.5 * C.astype(np.float64))
    # B = I: R = A
    A = rng.standard_normal((M, N)).astype(np.float32)
    eyeN = np.eye(N, dtype=np.float32)
    R, _ = oracle.gemm(M, N, N, 1.0, _buf(A, N), N, _buf(eyeN, N + 5), N + 5, 0.0, None, N)
    np.testing.assert_array_equal(R, A.astype(np.float64))
    # A = P (permutation): rows of B permuted, R[i] = B[p[i]]
    p = rng.permutation(M)
    P = np.zeros((M, M), np.float32)
    P[np.arange(M), p] = 1.0
    R, _ = oracle.gemm(M, N, M, 1.0, _buf(P, M), M, _buf(B, N), N, 0.0, None, N)
    np.testing.assert_array_equal(R, B[p].astype(np.float64))
    # B = Q (permutation on the right): columns of A permuted
    q = rng.permutation(N)
    Q = np.zeros((N, N), np.float32)
    Q[q, np.arange(N)] = 1.0
    R, _ = oracle.gemm(M, N, N, 1.0, _buf(A, N), N, _buf(Q, N), N, 0.0, None, N)
    np.testing.assert_array_equal(R, A[:, q].astype(np.float64))


def test_rectangular_identity_is_not_transposed():
    """A (2 x 3) times B (3 x 4) with one-hot entries: R_ij = A_i,k* B_k*,j picks
    a known element; a transposed or mis-indexed operand lands elsewhere."""
    M, N, K = 2, 4, 3
    for i, j, k in itertools.product(range(M), range(N), range(K)):
        A = np.zeros((M, K), np.float32)
        B = np.zeros((K, N), np.float32)
        A[i, k] = 3.0
        B[k, j] = 5.0
        R, _ = oracle.gemm(M, N, K, 1.0, _buf(A, K + 2), K + 2, _buf(B, N + 3), N + 3, 0.0, None, N)
        expect = np.zeros((M, N))
        expect[i, j] = 15.0
        np.testing.assert_array_equal(R, expect)


# ---------------------------------------------------------------- alpha / beta

def test_alpha_zero_does_not_read_A_or_B():
    M, N, K = 8, 9, 10
    A = np.full((M, K), np.nan, np.float32)
    B = np.full((K, N), np.inf, np.float32)
    C = np.arange(M * N, dtype=np.float32).reshape(M, N)
    R, G = oracle.gemm(M, N, K, 0.0, _buf(A, K), K, _buf(B, N), N, -0.5, _buf(C, N), N)
    np.testing.assert_array_equal(R, -0.5 * C.astype(np.float64))
    np.testing.assert_array_equal(G, 0.0)
    R, _ = oracle.gemm(M, N, K, 0.0, None, K, None, N, 0.0, None, N)
    np.testing.assert_array_equal(R, 0.0)


def test_beta_zero_does_not_read_C():
    M, N, K = 8, 9, 10
    rng = np.random.default_rng(5)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    C = np.full((M, N), np.nan, np.float32)
    R, _ = oracle.gemm(M, N, K, 1.0, _buf(A, K), K, _buf(B, N), N, 0.0, _buf(C, N), N)
    assert np.all(np.isfinite(R))
    np.testing.assert_allclose(R, A.astype(np.float64) @ B.astype(np.float64), rtol=1e-14, atol=1e-14)


def test_k_zero_and_empty():
    C = np.arange(12, dtype=np.float32).reshape(3, 4)
    R, G = oracle.gemm(3, 4, 0, 1.0, None, 1, None, 4, 2.0, _buf(C, 4), 4)
    np.testing.assert_array_equal(R, 2.0 * C)
    np.testing.assert_array_equal(G, 0.0)
    R, _ = oracle.gemm(0, 4, 3, 1.0, None, 3, None, 4, 1.0, None, 4)
    assert R.shape == (0, 4)
    R, _ = oracle.gemm(3, 0, 3, 1.0, None, 3, None, 1, 1.0, None, 1)
    assert R.shape == (3, 0)


def test_nan_propagates_when_read():
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 2), np.float32)
    A[1, 2] = np.nan
    R, _ = oracle.gemm(2, 2, 3, 1.0, _buf(A, 3), 3, _buf(B, 2), 2, 0.0, None, 2)
    assert np.all(np.isfinite(R[0])) and np.all(np.isnan(R[1]))


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("w", [wl.F32_SQUARE[0], wl.RAGGED_F32, wl.RAGGED_F16, wl.RAGGED_F16F32],
                         ids=lambda w: w.name)
def test_against_numpy_float64_matmul(w):
    """numpy's float64 matmul (dgemm) agrees with the oracle within the double
    summation error of either side."""
    A, B, C = wl.make(w)
    R, G = oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, w.dtype)
    a = wl.view(A, w.M, w.K, w.lda).astype(np.float64)
    b = wl.view(B, w.K, w.N, w.ldb).astype(np.float64)
    c = wl.view(C, w.M, w.N, w.ldc).astype(np.float64)
    ref = w.alpha * (a @ b) + w.beta * c
    mag = abs(w.alpha) * (np.abs(a) @ np.abs(b)) + abs(w.beta) * np.abs(c)
    assert np.all(np.abs(R - ref) <= 2 * (w.K + 3) * EPS53 * mag)
    np.testing.assert_allclose(G, np.abs(a) @ np.abs(b), rtol=2 * w.K * EPS53, atol=0)


def test_mixed_path_reads_fp32_C_and_half_inputs():
    """fp16 inputs with an fp32 C: the result is the fp32 oracle on the
    inputs widened to fp32 (exact) with the same fp32 C, bit for bit; C values
    below fp16's resolution change it."""
    rng = np.random.default_rng(19)
    M, N, K = 17, 23, 31
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float16)
    C = (rng.uniform(-1, 1, (M, N)) + 2.0 ** -20).astype(np.float32)
    Rm, Gm = oracle.gemm(M, N, K, -0.5, _buf(A, K), K, _buf(B, N), N, 1.25, _buf(C, N), N, "f16f32")
    R32, G32 = oracle.gemm(M, N, K, -0.5, _buf(A.astype(np.float32), K), K,
                           _buf(B.astype(np.float32), N), N, 1.25, _buf(C, N), N, "f32")
    np.testing.assert_array_equal(Rm, R32)
    np.testing.assert_array_equal(Gm, G32)
    Rh, _ = oracle.gemm(M, N, K, -0.5, _buf(A, K), K, _buf(B, N), N, 1.25,
                        _buf(C.astype(np.float16), N), N, "f16")
    assert not np.array_equal(Rm, Rh)


def test_f16_path_equals_f32_path_on_same_values():
    """fp16 inputs decode exactly; the fp16 oracle equals the fp32 oracle run
    on the same values widened to fp32."""
    rng = np.random.default_rng(9)
    M, N, K = 20, 30, 40
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float16)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float16)
    R16, G16 = oracle.gemm(M, N, K, 1.25, _buf(A, K), K, _buf(B, N), N, 0.75, _buf(C, N), N, "f16")
    R32, G32 = oracle.gemm(M, N, K, 1.25, _buf(A.astype(np.float32), K), K,
                           _buf(B.astype(np.float32), N), N, 0.75,
                           _buf(C.astype(np.float32), N), N, "f32")
    np.testing.assert_array_equal(R16, R32)
    np.testing.assert_array_equal(G16, G32)


@pytest.mark.parametrize("dtype", ["f32", "f16", "f16f32"])
def test_sampled_elements_small(dtype):
    rng = np.random.default_rng(4)
    M, N, K, lda, ldb, ldc = 23, 31, 45, 47, 36, 33
    tin, tc = (_NP[x] for x in wl.operand_types(dtype))
    A = _buf(rng.standard_normal((M, K)).astype(tin), lda)
    B = _buf(rng.standard_normal((K, N)).astype(tin), ldb)
    C = _buf(rng.standard_normal((M, N)).astype(tc), ldc, 5.0)
    for alpha, beta in [(1.5, -0.75), (0.0, 2.0), (-1.0, 0.0)]:
        R, G = oracle.gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype)
        rows, cols = wl.sample_positions(M, N, 200, 3)
        r, g = oracle.gemm_elems(rows, cols, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype)
        np.testing.assert_array_equal(r, R[rows, cols])
        np.testing.assert_array_equal(g, G[rows, cols])


def test_sampled_elements_match_full():
    w = wl.RAGGED_F32
    A, B, C = wl.make(w)
    R, G = oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    rows, cols = wl.sample_positions(w.M, w.N, 300, 1)
    r, g = oracle.gemm_elems(rows, cols, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    np.testing.assert_array_equal(r, R[rows, cols])
    np.testing.assert_array_equal(g, G[rows, cols])
    w = wl.RAGGED_F16
    A, B, C = wl.make(w)
    R, G = oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, "f16")
    r, g = oracle.gemm_elems(rows, cols, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, "f16")
    np.testing.assert_array_equal(r, R[rows, cols])
    np.testing.assert_array_equal(g, G[rows, cols])


# ---------------------------------------------------------------- whole-matrix checks

def test_checksum_and_freivalds_agree_with_full_result():
    w = wl.RAGGED_F32
    A, B, C = wl.make(w)
    R, G = oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    exp, mag = oracle.checksum(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    assert abs(R.sum() - exp) <= 1e-12 * mag
    x = np.random.default_rng(2).choice([-1.0, 1.0], size=w.N)
    y, ymag = oracle.freivalds(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, x)
    assert np.all(np.abs(R @ x - y) <= 1e-12 * ymag)
    # A one-element corruption of R is visible to Freivalds' check.
    R2 = R.copy()
    R2[123, 456] += 1e-3
    assert np.max(np.abs(R2 @ x - y)) > 1e-6


# ---------------------------------------------------------------- binary16

def test_half_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_half_encode_roundtrip_and_midpoints():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    back = oracle.round_f16(vals[finite])
    np.testing.assert_array_equal(back, bits[finite])
    # midpoints between consecutive positive finite halves round to the even one
    pos = np.arange(0, 0x7bff, dtype=np.uint16)           # 0 .. largest-1
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                                     # exact in double
    got = oracle.round_f16(mid)
    expect = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    np.testing.assert_array_equal(got, expect)
    np.testing.assert_array_equal(oracle.round_f16(-mid), expect | 0x8000)
    # just above / below a midpoint go to the nearer neighbour
    np.testing.assert_array_equal(oracle.round_f16(np.nextafter(mid, np.inf)), pos + 1)
    np.testing.assert_array_equal(oracle.round_f16(np.nextafter(mid, -np.inf)), pos)


def test_half_encode_random_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
                        rng.uniform(-70000, 70000, 50000)])
    ours = oracle.round_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_half_encode_specials():
    cases = [
        (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e6, 0x7C00), (np.inf, 0x7C00),
        (-65520.0, 0xFC00), (0.0, 0x0000), (-0.0, 0x8000), (2.0 ** -24, 0x0001),
        (2.0 ** -25, 0x0000), (3 * 2.0 ** -26, 0x0001), (3 * 2.0 ** -25, 0x0002),
        (2.0 ** -14, 0x0400), (2.0 ** -14 - 2.0 ** -25, 0x0400), (1.0, 0x3C00),
        (1 + 3 * 2.0 ** -11, 0x3C02),         # tie -> even (1 + 2^-9)
        (1 + 2.0 ** -11, 0x3C00),             # tie -> even (1)
        (1 + 0.75 * 2.0 ** -10, 0x3C01),      # nearer neighbour
    ]
    for x, b in cases:
        assert int(oracle.round_f16(np.array([x]))[0]) == b, (x, hex(b))
    assert int(oracle.round_f16(np.array([np.nan]))[0]) & 0x7C00 == 0x7C00


# ---------------------------------------------------------------- the bound

def _fp32_sequential(A, B, alpha, beta, C):
    """fp32 GEMM with one rounding per multiply-add, k ascending (numpy float32)."""
    acc = np.zeros((A.shape[0], B.shape[1]), np.float32)
    for k in range(A.shape[1]):
        acc = (acc + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    return (np.float32(alpha) * acc + np.float32(beta) * C).astype(np.float32)


def test_tolerance_admits_fp32_and_rejects_reduced_precision():
    rng = np.random.default_rng(21)
    M, N, K = 48, 40, 512
    A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    alpha, beta = 1.0, 0.5
    R, G = oracle.gemm(M, N, K, alpha, _buf(A, K), K, _buf(B, N), N, beta, _buf(C, N), N)
    tol = oracle.tolerance(G, np.abs(C), alpha, beta, K, R, "f32")
    ok, worst, _ = oracle.compare(_fp32_sequential(A, B, alpha, beta, C), R, tol)
    assert ok and worst < 0.5
    # operands truncated to bfloat16-like 8 significant bits must fail
    def trunc(x):
        return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    ok, worst, _ = oracle.compare(_fp32_sequential(trunc(A), trunc(B), alpha, beta, C), R, tol)
    assert not ok and worst > 2
    # fp16 output: RNE of R passes, a 2-ulp error fails somewhere
    R16 = oracle.round_f16(R)
    tol16 = oracle.tolerance(G, np.abs(C), alpha, beta, K, R, "f16")
    assert oracle.compare(R16, R, tol16)[0]
    bad = (R16.astype(np.int32) + 2).astype(np.uint16)
    assert not oracle.compare(bad, R, tol16)[0]


def test_compare_nan_and_inf_handling():
    R = np.array([1.0, np.nan, np.inf])
    tol = np.array([1e-6, 1e-6, 1e-6])
    assert oracle.compare(np.array([1.0, np.nan, np.inf], np.float32), R, tol)[0]
    assert not oracle.compare(np.array([np.nan, np.nan, np.inf], np.float32), R, tol)[0]
    assert not oracle.compare(np.array([1.0, 0.0, np.inf], np.float32), R, tol)[0]
    assert not oracle.compare(np.array([1.0, np.nan, -np.inf], np.float32), R, tol)[0]


# ---------------------------------------------------------------- tolerance, by hand

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _exact_term(t):
    """'c*2^e', '2^e' or a decimal number, as an exact Fraction."""
    t = t.strip()
    coef, _, powr = t.rpartition("*") if "^" in t else ("", "", t)
    if "^" in powr:
        base, e = powr.split("^")
        assert base == "2", t
        v = Fraction(2) ** int(e)
        return v * (Fraction(coef) if coef else 1)
    return Fraction(powr)


def _exact_sum(expr):
    return sum((_exact_term(t) for t in expr.split("+")), Fraction(0))


def _tolerance_rows():
    rows = []
    with open(os.path.join(GOLDEN, "tolerance.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("|")
            out, K, alpha, beta, G, Cabs, R = lhs.split()
            rows.append((out, int(K), *(float(_exact_term(x)) for x in (alpha, beta, G, Cabs, R)),
                         _exact_sum(rhs)))
    return rows


def test_tolerance_matches_hand_computed_values():
    """The bound at hand-worked points (tests/golden/tolerance.txt): K = 0,
    beta*C alone, a subnormal-range R, large |R|, a negative alpha, fp32 and
    fp16 outputs.  A wrong u_out, a dropped |beta||C|, eta or (1 + u_out)
    term, 4K in place of K, or K in place of max(K, 1) each miss one row."""
    rows = _tolerance_rows()
    assert len(rows) >= 9
    for out, K, alpha, beta, G, Cabs, R, expect in rows:
        got = oracle.tolerance(np.array([G]), np.array([Cabs]), alpha, beta, K, np.array([R]), out)
        got = Fraction(float(got[0]))
        assert abs(got - expect) <= expect * Fraction(1, 2 ** 50), (out, K, alpha, beta, G, Cabs, R,
                                                                   float(got), float(expect))


def test_compare_boundary_sign_and_shape():
    """An error exactly equal to the bound passes, one just above fails, in
    either direction; the worst ratio and its position are reported."""
    R = np.array([[1.0, 2.0], [3.0, 4.0]])
    tol = np.full((2, 2), 2.0 ** -20)
    at = R + np.array([[0.0, 2.0 ** -20], [0.0, -2.0 ** -20]])
    ok, worst, idx = oracle.compare(at, R, tol)
    assert ok and worst == 1.0 and idx in ((0, 1), (1, 1))
    over = R.copy()
    over[1, 0] -= 2.0 ** -19        # below R by twice the bound
    ok, worst, idx = oracle.compare(over, R, tol)
    assert not ok and worst == 2.0 and idx == (1, 0)
    over = R.copy()
    over[0, 0] += 2.0 ** -19
    assert not oracle.compare(over, R, tol)[0]
    assert oracle.compare(np.zeros((0, 3)), np.zeros((0, 3)), np.zeros((0, 3)))[0]


# A 2 x 2 by 2 x 3 product worked out by hand for the whole-matrix checks:
#   A = [[1, -2], [3, 4]], B = [[1, -1, 2], [0, 3, -1]], C = [[1, -1, 0], [2, 0, 1]],
#   alpha = 2, beta = -3.  AB = [[1, -7, 4], [3, 9, 2]] (sum 12), sum C = 3:
#   checksum = 2*12 - 3*3 = 15;  magnitude = 2 * (colsum|A| . rowsum|B|)
#   + 3 * sum|C| = 2 * ([4, 6] . [4, 4]) + 3 * 5 = 80 + 15 = 95.
#   x = [1, -1, 1]: ABx = [12, -4], Cx = [2, 3], y = 2*ABx - 3*Cx = [18, -17];
#   |B||x| = [4, 4], |A|[4, 4] = [12, 28], |C||x| = [2, 3]:
#   magnitude = 2*[12, 28] + 3*[2, 3] = [30, 65].
_HA = np.array([[1, -2], [3, 4]], np.float32)
_HB = np.array([[1, -1, 2], [0, 3, -1]], np.float32)
_HC = np.array([[1, -1, 0], [2, 0, 1]], np.float32)


@pytest.mark.parametrize("dtype", ["f32", "f16", "f16f32"])
def test_checksum_and_freivalds_hand_computed(dtype):
    tin, tc = (_NP[x] for x in wl.operand_types(dtype))
    A = _buf(_HA.astype(tin), 3)
    B = _buf(_HB.astype(tin), 5)
    C = _buf(_HC.astype(tc), 4)
    exp, mag = oracle.checksum(2, 3, 2, 2.0, A, 3, B, 5, -3.0, C, 4, dtype)
    assert (exp, mag) == (15.0, 95.0)
    y, ymag = oracle.freivalds(2, 3, 2, 2.0, A, 3, B, 5, -3.0, C, 4, np.array([1.0, -1.0, 1.0]),
                               dtype)
    np.testing.assert_array_equal(y, [18.0, -17.0])
    np.testing.assert_array_equal(ymag, [30.0, 65.0])
    # beta = 0: C is neither summed nor counted (its buffer may be absent)
    exp, mag = oracle.checksum(2, 3, 2, 2.0, A, 3, B, 5, 0.0, None, 4, dtype)
    assert (exp, mag) == (24.0, 80.0)
