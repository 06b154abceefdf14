"""GPU parity of gemm_f32 / gemm_f16 against the CPU oracle, called through
the C ABI.  Tolerance: |err| <= (1+u_out)*4*max(K,1)*2^-24*(|alpha|G + |beta||C|)
+ u_out*|R| + eta_out (oracle.tolerance), elementwise; bitwise equality where
every partial sum is exact."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as wl
from gemm_harness import (assert_pads_unchanged, bits, check, check_sampled, colmajor_buf,
                          colmajor_view, exact_expected,
                          note, np_in, np_out, run, run_colmajor)

pytestmark = pytest.mark.gpu

# "f16f32": fp16 A and B with an fp32 C and result (gemm_f16f32).
DTYPES = ["f32", "f16", "f16f32"]


def _t(dtype):
    """Storage type of A and B."""
    return np_in(dtype)


def _tc(dtype):
    """Storage type of C and of the result."""
    return np_out(dtype)


def _w_run_check(w, label=None):
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, w.name)
    assert rc == 0
    return check(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, out,
                 label or w.name)


# ---------------------------------------------------------------- workloads

def test_f32_256():
    _w_run_check(wl.F32_256)


@pytest.mark.parametrize("n", [256, 512, 1024, 2048])
def test_f32_square_full_oracle(n):
    _w_run_check(wl.square(n, seeds=(2, 3, 4)))


@pytest.mark.parametrize("w", [wl.RAGGED_F32, wl.RAGGED_F16, wl.RAGGED_F16F32], ids=lambda w: w.name)
def test_ragged_padded_unaligned(w):
    """1000 x 3000 x 517, lda=530, ldb=3005, ldc=3003: unaligned leading
    dimensions (scalar loads), all three tails, NaN in the pads of A and B,
    sentinels in the pad of C."""
    _w_run_check(w)


def _plan(w):
    import dense_gemm_fp32_amd as dg
    rc, text = dg.gemm_describe(w.dtype, w.M, w.N, w.K, w.alpha, 4096, w.lda, 4096, w.ldb, w.beta,
                                4096, w.ldc)
    assert rc == 0
    return text


@pytest.mark.parametrize("w", [wl.F32_4096, wl.F16_4096, wl.F16F32_4096], ids=lambda w: w.name)
def test_headline_4096_every_element(w):
    """The 4096^3 workloads (fp32 with beta = 0; fp16 and fp16-in/fp32-out
    with beta = 0.5), in the configuration the benchmark times, compared with
    the full oracle element by element: all 16.7 million outputs."""
    plan = _plan(w)
    assert "256x256" in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("n,tile,whole", [(1152, "64x64x64 4 waves 2 slots", 0),
                                          (1408, "64x64x64 4 waves 2 slots", 0),
                                          (1536, "64x64x32 4 waves", 512),
                                          (1664, "64x64x32 4 waves", 0),
                                          (1792, "64x64x32 4 waves", 768),
                                          (1920, "128x64x32 4 waves", 0)])
def test_f32_sweep_four_wave_tile_full_oracle(n, tile, whole):
    """Sweep sizes (beta = 1) whose plan is a four-wave tile, K unsplit: the
    64x64 tile of 32x32 waves (one to three and a third tiles per CU; up to
    two per CU in 64-k steps) or the 128x64 tile of 64x32 waves (past that,
    up to 2 per CU), every element against the oracle.
    1536^3 (576 tiles) and 1792^3 (784) leave a small last round, whose K
    steps run Stream-K behind the whole ones."""
    w = wl.sweep(n)
    plan = _plan(w)
    assert tile in plan and "split" not in plan, plan
    if whole:
        assert "stream-K after %d whole tiles" % whole in plan, plan
    else:
        assert "stream-K" not in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("n,blocks", [(3200, "mfma32x32x16"), (3584, "mfma16x16x32")])
def test_f16_large_tile_block_shape_by_size_sampled(n, blocks):
    """fp16 sizes whose 256x256 tiles fill less than every CU: 32x32x16
    blocks below three quarters of the CUs (3200^3, 169 tiles), 16x16x32 from
    there (3584^3, 196 tiles); sampled rows against the oracle, with rows of
    the last tile row."""
    w = wl.Workload("f16_%d_beta0.5" % n, "f16", n, n, n, n, n, n, 1.0, 0.5, "uniform", "uniform",
                    (3, 4, 5))
    plan = _plan(w)
    assert "256x256x64" in plan and blocks in plan, plan
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                  "%s (%s)" % (w.name, plan))
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=16, seed=n, extra_rows=[n - 1, n - 200])


@pytest.mark.parametrize("shape", [(896, 896, 896), (1024, 768, 1024), (600, 1600, 800),
                                   (512, 1024, 256), (64, 8192, 512)])
def test_f32_under_one_round_four_wave_tile_full_oracle(shape):
    """Grids under one round of 64x64 tiles where the size rule takes that
    tile with four waves, unsplit, in place of the 32x32 tile (896^3, 600 x
    1600 x 800), of a K split (1024 x 768 x 1024) or of a larger tile that
    would leave most CUs idle (512 x 1024 x 256, 64 x 8192 x 512): every
    element against the oracle (beta = 1)."""
    M, N, K = shape
    w = wl.Workload("quad_%dx%dx%d" % shape, "f32", M, N, K, K, N, N, 1.0, 1.0, "uniform",
                    "uniform", (91, 92, 93))
    plan = _plan(w)
    assert "64x64x64 4 waves 2 slots" in plan and "split" not in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("n", [2944, 3584])
def test_f32_sweep_mid_sizes_sampled(n):
    """Sweep sizes whose chosen plans split K: 2944^3 and 3584^3 (the last,
    partly filled round of tiles split), with
    beta = 1, on sampled rows that include one row of each of the last eight
    tile rows (where the split leftover tiles lie), the checksum and
    Freivalds' check."""
    w = wl.sweep(n)
    plan = _plan(w)
    assert "split-K" in plan, plan
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                  "%s (%s)" % (w.name, plan))
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=24, seed=n,
                  extra_rows=[n - 1 - 128 * i - 37 for i in range(8)])


def test_f32_sweep_endpoints_sampled():
    """The size sweep's first size with beta = 1 (accumulating into C)."""
    w = wl.sweep(1024)
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, w.name)
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=32)


# ---------------------------------------------------------------- tails

TAIL_DIMS = [1, 2, 7, 31, 33, 64, 127, 129, 255, 257]


@pytest.mark.parametrize("dtype", DTYPES)
def test_tails_brute_force(dtype):
    """Every combination of small and tile-crossing M, N, K (aligned and
    unaligned leading dimensions) against the full oracle."""
    rng = np.random.default_rng(17)
    t = _t(dtype)
    combos = list(itertools.product(TAIL_DIMS, repeat=3))
    rng.shuffle(combos)
    for idx, (M, N, K) in enumerate(combos[:120]):
        pad = int(rng.integers(0, 9))
        lda, ldb, ldc = K + pad, N + (pad + 3) % 9, N + (2 * pad) % 9
        alpha = float(t(rng.uniform(0.5, 2)))
        beta = [0.0, 1.0, -0.5][idx % 3]
        A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(t), lda, np.nan)
        B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(t), ldb, np.nan)
        C = wl.pad(rng.uniform(-1, 1, (M, N)).astype(_tc(dtype)), ldc, wl.C_PAD_SENTINEL)
        rc, out = run(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, "tail")
        assert rc == 0
        check(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out,
              "tail M=%d N=%d K=%d ld=%d,%d,%d" % (M, N, K, lda, ldb, ldc))


# ---------------------------------------------------------------- exactness

@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (-1.0, 1.0), (2.0, -2.0), (1.0, 0.5)])
def test_f32_small_integers_exact(alpha, beta):
    """A, B, C in {-8..8}, K = 1000: every partial sum is an integer below
    2^24, so the result must equal the correctly rounded value bit for bit."""
    M, N, K = 300, 260, 1000
    A = wl.small_ints(M, K, -8, 8, 1, "f32")
    B = wl.small_ints(K, N, -8, 8, 2, "f32")
    C = wl.small_ints(M, N, -8, 8, 3, "f32")
    A, B, C = A.reshape(-1), B.reshape(-1), C.reshape(-1)
    rc, out = run("f32", M, N, K, alpha, A, K, B, N, beta, C, N, "ints")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, alpha, A, K, B, N, beta, C, N)
    assert np.array_equal(bits(out.reshape(M, N), "f32"), bits(exact_expected("f32", R), "f32"))


def test_f32_full_precision_operands_exact():
    """A = odd integers up to 4095 (12 significant bits), B in {-1, 0, 1}:
    exact in fp32 for K = 4096, but any rounding of the operands below 12
    significant bits (tf32 / bf16-style) breaks equality.  Both operand roles."""
    M, N, K = 256, 192, 4096
    A = wl.odd_ints(M, K, 4095, 5).reshape(-1)
    B = wl.small_ints(K, N, -1, 1, 6, "f32").reshape(-1)
    rc, out = run("f32", M, N, K, 1.0, A, K, B, N, 0.0, np.zeros(M * N, np.float32), N, "odd")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, 1.0, A, K, B, N, 0.0, None, N)
    assert np.all(np.abs(R) < 2 ** 24)
    assert np.array_equal(bits(out.reshape(M, N), "f32"), bits(exact_expected("f32", R), "f32"))
    # transposed roles: B holds the 12-bit values
    A2 = wl.small_ints(M, K, -1, 1, 7, "f32").reshape(-1)
    B2 = wl.odd_ints(K, N, 4095, 8).reshape(-1)
    rc, out = run("f32", M, N, K, 1.0, A2, K, B2, N, 0.0, np.zeros(M * N, np.float32), N, "odd2")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, 1.0, A2, K, B2, N, 0.0, None, N)
    assert np.array_equal(bits(out.reshape(M, N), "f32"), bits(exact_expected("f32", R), "f32"))


@pytest.mark.parametrize("beta", [0.0, 1.0, -1.0, 2.0])
def test_f16_small_integers_exact(beta):
    """A, B in {-3..3}, K = 200, C in {-8..8}: |R| <= 1816 + 16 is an integer,
    exact in fp16, so the output must equal it bit for bit."""
    M, N, K = 200, 280, 200
    A = wl.small_ints(M, K, -3, 3, 11, "f16").reshape(-1)
    B = wl.small_ints(K, N, -3, 3, 12, "f16").reshape(-1)
    C = wl.small_ints(M, N, -8, 8, 13, "f16").reshape(-1)
    rc, out = run("f16", M, N, K, 1.0, A, K, B, N, beta, C, N, "f16ints")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, 1.0, A, K, B, N, beta, C, N, "f16")
    assert np.all(np.abs(R) <= 2048)
    assert np.array_equal(bits(out, "f16"), oracle.round_f16(R).reshape(-1))


@pytest.mark.parametrize("beta", [0.0, 1.0, -0.75])
def test_f16f32_small_integers_and_fine_C_exact(beta):
    """fp16 A, B in {-8..8}, K = 1000, fp32 C = integers plus multiples of
    2^-10: every partial sum and the result are exact in fp32 (not in fp16), so
    the output must equal the correctly rounded value bit for bit -- an output
    rounded through half, or a C read as half, cannot."""
    M, N, K = 260, 300, 1000
    A = wl.small_ints(M, K, -8, 8, 21, "f16").reshape(-1)
    B = wl.small_ints(K, N, -8, 8, 22, "f16").reshape(-1)
    C = (wl.small_ints(M, N, -64, 64, 23, "f32")
         + wl.small_ints(M, N, -512, 512, 24, "f32") / 1024.0).astype(np.float32).reshape(-1)
    rc, out = run("f16f32", M, N, K, 1.0, A, K, B, N, beta, C, N, "f16f32ints")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, 1.0, A, K, B, N, beta, C, N, "f16f32")
    assert np.array_equal(bits(out, "f16f32"), bits(exact_expected("f16f32", R).reshape(-1), "f16f32"))


def test_f16_output_rounding_is_nearest_even():
    """K = 2, A = [1, 3*2^-11], B = [1, 1]^T: the fp32 accumulator is exactly
    1 + 3*2^-11, halfway between halves 1+2^-10 and 1+2^-9; ties-to-even gives
    1 + 2^-9 (round-toward-zero would give 1 + 2^-10).  1 + 0.75*2^-10 is
    not a tie and goes to 1 + 2^-10."""
    A = np.array([1.0, 3 * 2.0 ** -11, 1.0, 0.75 * 2.0 ** -10], np.float16)
    B = np.array([1.0, 1.0], np.float16)
    C = np.zeros(2, np.float16)
    rc, out = run("f16", 2, 1, 2, 1.0, A, 2, B, 1, 0.0, C, 1, "rne")
    assert rc == 0
    got = bits(out, "f16")
    assert int(got[0]) == 0x3C02, hex(got[0])
    assert int(got[1]) == 0x3C01, hex(got[1])
    # overflow: 2 * 65504 rounds to +inf; -65520 ties to -inf
    A = np.array([65504.0, 65504.0, -32752.0, -32768.0], np.float16)
    B = np.array([1.0, 1.0], np.float16)
    rc, out = run("f16", 2, 1, 2, 1.0, A, 2, B, 1, 0.0, C, 1, "ovf")
    assert rc == 0
    got = bits(out, "f16")
    assert int(got[0]) == 0x7C00 and int(got[1]) == 0xFC00, [hex(g) for g in got]


# ---------------------------------------------------------------- special matrices

@pytest.mark.parametrize("dtype", DTYPES)
def test_identity_and_permutation_bitwise(dtype):
    t, tc = _t(dtype), _tc(dtype)
    rng = np.random.default_rng(31)
    M, N = 300, 200
    B = rng.uniform(-1, 1, (M, N)).astype(t)
    eye = np.eye(M, dtype=t)
    C0 = np.zeros(M * N, tc)
    rc, out = run(dtype, M, N, M, 1.0, eye.reshape(-1), M, B.reshape(-1), N, 0.0, C0, N, "A=I")
    assert rc == 0 and np.array_equal(bits(out, dtype), bits(B.reshape(-1).astype(tc), dtype))
    A = rng.uniform(-1, 1, (M, N)).astype(t)
    eyeN = np.eye(N, dtype=t)
    rc, out = run(dtype, M, N, N, 1.0, A.reshape(-1), N, eyeN.reshape(-1), N, 0.0, C0, N, "B=I")
    assert rc == 0 and np.array_equal(bits(out, dtype), bits(A.reshape(-1).astype(tc), dtype))
    p = rng.permutation(M)
    P = np.zeros((M, M), t)
    P[np.arange(M), p] = 1
    rc, out = run(dtype, M, N, M, 1.0, P.reshape(-1), M, B.reshape(-1), N, 0.0, C0, N, "A=P")
    assert rc == 0 and np.array_equal(bits(out, dtype), bits(B[p].reshape(-1).astype(tc), dtype))


# ---------------------------------------------------------------- alpha / beta

@pytest.mark.parametrize("dtype", DTYPES)
def test_alpha_zero_ignores_A_and_B(dtype):
    t, tc = _t(dtype), _tc(dtype)
    M, N, K = 130, 70, 90
    A = np.full(M * K, np.nan, t)
    B = np.full(K * N, np.inf, t)
    C = np.random.default_rng(1).uniform(-1, 1, M * N).astype(tc)
    rc, out = run(dtype, M, N, K, 0.0, A, K, B, N, -0.5, C, N, "alpha0")
    assert rc == 0
    expect = (np.float32(-0.5) * C.astype(np.float32)).astype(tc)
    assert np.array_equal(bits(out, dtype), bits(expect, dtype))
    # alpha = 0 and beta = 0: exact zeros, C (NaN here) not read
    Cn = np.full(M * N, np.nan, tc)
    rc, out = run(dtype, M, N, K, 0.0, A, K, B, N, 0.0, Cn, N, "alpha0beta0")
    assert rc == 0 and np.all(out == 0)
    # alpha = 0, beta = 1: C unchanged bit for bit (nothing launched)
    rc, out = run(dtype, M, N, K, 0.0, None, K, None, N, 1.0, C, N, "alpha0beta1")
    assert rc == 0 and np.array_equal(bits(out, dtype), bits(C, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_beta_zero_ignores_C(dtype):
    t = _t(dtype)
    M, N, K = 257, 129, 65
    rng = np.random.default_rng(2)
    A = rng.uniform(-1, 1, M * K).astype(t)
    B = rng.uniform(-1, 1, K * N).astype(t)
    Cn = np.full(M * N, np.nan, _tc(dtype))
    rc, out = run(dtype, M, N, K, 1.0, A, K, B, N, 0.0, Cn, N, "beta0")
    assert rc == 0 and np.all(np.isfinite(out.astype(np.float64)))
    check(dtype, M, N, K, 1.0, A, K, B, N, 0.0, Cn, N, out, "beta0")


@pytest.mark.parametrize("dtype", DTYPES)
def test_k_zero_scales_C(dtype):
    t = _t(dtype)
    M, N = 100, 300
    C = np.random.default_rng(3).uniform(-1, 1, M * (N + 4)).astype(_tc(dtype))
    rc, out = run(dtype, M, N, 0, 1.0, None, 1, None, N, 2.0, C, N + 4, "k0")
    assert rc == 0
    check(dtype, M, N, 0, 1.0, None, 1, None, N, 2.0, C, N + 4, out, "k0")


# ---------------------------------------------------------------- determinism, paths

@pytest.mark.parametrize("dtype", DTYPES)
def test_bitwise_deterministic_and_scalar_path_agrees(dtype):
    """Two identical calls give identical bits; forcing element-wise loads
    changes only how data moves, not the summation order, so the forced-scalar
    result is bitwise equal too."""
    import dense_gemm_fp32_amd as dg
    t = _t(dtype)
    M, N, K = 700, 900, 600
    rng = np.random.default_rng(4)
    A = rng.standard_normal(M * K).astype(t)
    B = rng.standard_normal(K * N).astype(t)
    C = rng.standard_normal(M * N).astype(_tc(dtype))
    rc1, o1 = run(dtype, M, N, K, 1.5, A, K, B, N, -0.75, C, N, "det1")
    rc2, o2 = run(dtype, M, N, K, 1.5, A, K, B, N, -0.75, C, N, "det2")
    assert rc1 == rc2 == 0 and np.array_equal(bits(o1, dtype), bits(o2, dtype))
    prev = dg.gemm_set_load_mode(1)
    try:
        rc3, o3 = run(dtype, M, N, K, 1.5, A, K, B, N, -0.75, C, N, "scalar")
    finally:
        dg.gemm_set_load_mode(prev)
    assert rc3 == 0 and np.array_equal(bits(o1, dtype), bits(o3, dtype))
    check(dtype, M, N, K, 1.5, A, K, B, N, -0.75, C, N, o1, "det")


def test_torch_wrapper_matches_raw_call():
    import torch
    import dense_gemm_fp32_amd as dg
    g = torch.Generator().manual_seed(0)
    A = torch.rand(333, 444, generator=g).cuda()
    B = torch.rand(444, 555, generator=g).cuda()
    C = torch.zeros(333, 555).cuda()
    dg.gemm(A, B, C, 1.0, 0.0)
    torch.cuda.synchronize()
    R, G = oracle.gemm(333, 555, 444, 1.0, A.cpu().numpy().reshape(-1), 444,
                       B.cpu().numpy().reshape(-1), 555, 0.0, None, 555)
    tol = oracle.tolerance(G, 0.0, 1.0, 0.0, 444, R)
    assert oracle.compare(C.cpu().numpy(), R, tol)[0]


# ---------------------------------------------------------------- fp16 load paths

# Leading dimensions that are multiples of 8 halves (16-byte rows) send the
# fp16 kernel's interior tiles through direct global->LDS loads; these shapes
# put every edge case of that path in play: rows past M (clamped reads), a
# column edge with N % 8 == 0 (clamped chunks) and != 0 (that tile column
# takes the masked register path while the others stay direct), a partial K
# step (done first, masked), K shorter than one step, and exact multiples.
F16_PATH_SHAPES = [
    # M,    N,   K,  lda, ldb, ldc
    (300, 264, 100, 104, 264, 264),
    (257, 512, 64, 64, 512, 520),
    (600, 530, 96, 96, 536, 536),
    (256, 256, 17, 24, 256, 256),
    (513, 776, 1000, 1000, 776, 784),
    (64, 1024, 544, 552, 1024, 1024),
]


@pytest.mark.parametrize("dtype", ["f16", "f16f32"])
@pytest.mark.parametrize("shape", F16_PATH_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_direct_path_edges_match_oracle_and_staged_path(shape, dtype):
    import dense_gemm_fp32_amd as dg
    M, N, K, lda, ldb, ldc = shape
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(np.float16), lda, np.nan)
    B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(np.float16), ldb, np.nan)
    C = wl.pad(rng.uniform(-1, 1, (M, N)).astype(_tc(dtype)), ldc, wl.C_PAD_SENTINEL)
    rc, out_direct = run(dtype, M, N, K, 1.25, A, lda, B, ldb, -0.5, C, ldc, "f16 direct")
    assert rc == 0
    check(dtype, M, N, K, 1.25, A, lda, B, ldb, -0.5, C, ldc, out_direct, "direct %s" % (shape,))
    prev = dg.gemm_set_load_mode(1)
    try:
        rc, out_staged = run(dtype, M, N, K, 1.25, A, lda, B, ldb, -0.5, C, ldc, "f16 staged")
    finally:
        dg.gemm_set_load_mode(prev)
    assert rc == 0
    # same LDS layout and summation order on both paths: identical bits
    assert np.array_equal(bits(out_direct, dtype), bits(out_staged, dtype))


def test_f16_nan_in_a_row_past_m_is_not_read():
    """Rows past M are clamped to row M-1 on the direct path: a NaN placed in
    the memory right after A's last row must not reach C."""
    M, N, K = 200, 256, 64
    rng = np.random.default_rng(5)
    A = np.concatenate([rng.uniform(-1, 1, M * K).astype(np.float16),
                        np.full(64 * K, np.nan, np.float16)])
    B = rng.uniform(-1, 1, K * N).astype(np.float16)
    C = np.zeros(M * N, np.float16)
    rc, out = run("f16", M, N, K, 1.0, A, K, B, N, 0.0, C, N, "rows past M")
    assert rc == 0
    check("f16", M, N, K, 1.0, A, K, B, N, 0.0, C, N, out, "rows past M")


# ---------------------------------------------------------------- tile table

from contextlib import contextmanager


@contextmanager
def tile_config(cfg):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_tile_config(cfg)
    try:
        yield
    finally:
        dg.gemm_set_tile_config(prev)


TABLE_SHAPES = [
    # M,    N,   K,  lda, ldb, ldc   (aligned: direct loads with every edge)
    (300, 264, 100, 104, 264, 264),
    (600, 640, 96, 96, 648, 640),
    # unaligned leading dimensions: register-staged path
    (257, 530, 77, 77, 533, 531),
]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10],
                         ids=["large", "medium", "small", "tiny", "medium-bunched", "f32-256x256",
                              "f32-64x64-four-waves", "f32-128x64-four-waves",
                              "f32-64x64-four-waves-k64", "f32-32x32-k64"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_every_tile_configuration_matches_oracle(dtype, cfg):
    t = _t(dtype)
    for shape in TABLE_SHAPES:
        M, N, K, lda, ldb, ldc = shape
        rng = np.random.default_rng(M + 3 * N + 7 * K + cfg)
        A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(t), lda, np.nan)
        B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(t), ldb, np.nan)
        C = wl.pad(rng.uniform(-1, 1, (M, N)).astype(_tc(dtype)), ldc, wl.C_PAD_SENTINEL)
        with tile_config(cfg):
            rc, out = run(dtype, M, N, K, 0.75, A, lda, B, ldb, 1.5, C, ldc, "cfg%d" % cfg)
        assert rc == 0
        check(dtype, M, N, K, 0.75, A, lda, B, ldb, 1.5, C, ldc, out, "cfg %d %s" % (cfg, shape))


@pytest.mark.parametrize("dtype", DTYPES)
def test_large_tiles_with_edges_sampled(dtype):
    """Large-tile configuration picked by size, with all three edges and
    aligned leading dimensions (direct loads with clamping), checked on
    sampled rows, the checksum and Freivalds' product check."""
    w = wl.Workload("edges_large_" + dtype, dtype, 4100, 4104, 1000, 1000, 4104, 4112, 1.25, -0.5,
                    "uniform", "uniform", (21, 22, 23))
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, w.name)
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=24)


def test_f32_sweep_largest_size_sampled():
    """The size sweep's largest size, 12800^3 with beta = 1 (large-tile
    configuration, direct loads), on sampled rows, the checksum and
    Freivalds' check."""
    w = wl.sweep(12800)
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, w.name)
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=16)


# ---------------------------------------------------------------- randomized shapes

from hypothesis import HealthCheck, given, settings, strategies as st


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(dtype=st.sampled_from(DTYPES),
       M=st.integers(1, 300), N=st.integers(1, 300), K=st.integers(1, 300),
       pads=st.tuples(st.integers(0, 9), st.integers(0, 9), st.integers(0, 9)),
       alpha=st.sampled_from([1.0, -0.5, 2.0, 0.25]),
       beta=st.sampled_from([0.0, 1.0, -1.5, 0.5]),
       cfg=st.sampled_from([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10]),
       pack=st.sampled_from([0, 2]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_shapes_match_oracle(dtype, M, N, K, pads, alpha, beta, cfg, pack, seed):
    """Random small shapes (every tail residue of every tile size is
    reachable), random row padding (aligned and unaligned leading
    dimensions), alpha/beta, forced tile configurations, and operand copies
    by size (none at these sizes) or forced."""
    t = _t(dtype)
    rng = np.random.default_rng(seed)
    lda, ldb, ldc = K + pads[0], N + pads[1], N + pads[2]
    A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(t), lda, np.nan)
    B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(t), ldb, np.nan)
    C = wl.pad(rng.uniform(-1, 1, (M, N)).astype(_tc(dtype)), ldc, wl.C_PAD_SENTINEL)
    with tile_config(cfg), pack_mode(pack):
        rc, out = run(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      "hyp cfg%d pack%d" % (cfg, pack))
    assert rc == 0
    check(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out,
          "random %s M=%d N=%d K=%d ld=%d,%d,%d cfg=%d pack=%d" % (dtype, M, N, K, lda, ldb, ldc,
                                                                 cfg, pack))


# ---------------------------------------------------------------- split K

@contextmanager
def split_mode(mode):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_split(mode)
    try:
        yield
    finally:
        dg.gemm_set_split(prev)


SPLIT_SHAPES = [
    # M,    N,    K,  lda,  ldb,  ldc    (aligned: direct loads; K tail)
    (300, 264, 1000, 1000, 264, 264),
    # unaligned leading dimensions (register-staged loads), all three tails
    (257, 530, 777, 781, 533, 531),
    # deep K, little M x N
    (64, 72, 4096, 4096, 72, 80),
]


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("dtype", DTYPES)
def test_split_k_matches_oracle(dtype, splits):
    """Forced split K (each chunk's fp32 sums to a pooled workspace, then one
    ordered reduction with alpha, beta and the output rounding) against the
    full oracle; beta = 0 with a NaN-filled C checks that C stays write-only."""
    t, tc = _t(dtype), _tc(dtype)
    for idx, shape in enumerate(SPLIT_SHAPES):
        M, N, K, lda, ldb, ldc = shape
        rng = np.random.default_rng(M + 5 * N + 11 * K + splits)
        A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(t), lda, np.nan)
        B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(t), ldb, np.nan)
        beta = [-0.5, 0.0, 1.0][idx % 3]
        cvals = rng.uniform(-1, 1, (M, N)).astype(tc) if beta != 0 else np.full((M, N), np.nan, tc)
        C = wl.pad(cvals, ldc, wl.C_PAD_SENTINEL)
        with split_mode(splits):
            rc, out = run(dtype, M, N, K, 1.25, A, lda, B, ldb, beta, C, ldc, "split%d" % splits)
        assert rc == 0
        check(dtype, M, N, K, 1.25, A, lda, B, ldb, beta, C, ldc, out,
              "split %d %s %s" % (splits, dtype, shape))


@pytest.mark.parametrize("w", [wl.RAGGED_F32, wl.RAGGED_F16, wl.RAGGED_F16F32], ids=lambda w: w.name)
def test_split_k_ragged_workload(w):
    """The ragged 1000 x 3000 x 517 workload (unaligned, NaN pads, C-pad
    sentinel) with K split in 4."""
    A, B, C = wl.make(w)
    with split_mode(4):
        rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc,
                      w.name + " split4")
    assert rc == 0
    check(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, out,
          w.name + " split4")


# Shapes that the size-based choice itself splits through its rules for wide,
# short problems and for unaligned (element-wise loaded) operands:
# (dtype, M, N, K, pad of lda / ldb / ldc, expected split in the plan).
CHOSEN_SPLIT_CASES = [
    ("f32", 2048, 384, 2048, (0, 0, 0), "split-K 5"),      # fewer 64x64 tiles than CUs, aligned
    ("f32", 1024, 1024, 4096, (0, 0, 0), "split-K 8"),     # deep K
    ("f32", 517, 3000, 1000, (13, 5, 3), "split-K 4"),     # unaligned
    ("f32", 2000, 2000, 1000, (13, 5, 3), "split-K 3"),
    ("f16", 1500, 1500, 1500, (13, 5, 3), "split-K 3"),
    ("f16", 517, 3000, 1000, (13, 5, 3), "split-K 4"),
    ("f16f32", 1000, 3000, 517, (13, 5, 3), "split-K 2"),
]


@pytest.mark.parametrize("case", CHOSEN_SPLIT_CASES, ids=lambda c: "%s_%dx%dx%d_pad%d" % (c[0], *c[1:4], c[4][0]))
def test_splits_chosen_by_rule_match_oracle(case):
    """The plan takes the expected split by itself (no tile or split switch;
    operand copies off, so unaligned operands keep their staged loads), with
    NaN pads and a C-pad sentinel, and matches the oracle element by
    element."""
    import dense_gemm_fp32_amd as dg
    dtype, M, N, K, (pa, pb, pc), want = case
    lda, ldb, ldc = K + pa, N + pb, N + pc
    rng = np.random.default_rng(M + 7 * N + 13 * K + pa)
    A = wl.pad(rng.standard_normal((M, K)).astype(_t(dtype)), lda, np.nan)
    B = wl.pad(rng.standard_normal((K, N)).astype(_t(dtype)), ldb, np.nan)
    C = wl.pad(rng.standard_normal((M, N)).astype(_tc(dtype)), ldc, wl.C_PAD_SENTINEL)
    base = 1 << 20
    with pack_mode(1):
        plan = dg.gemm_describe(dtype, M, N, K, 1.5, base, lda, base, ldb, -0.75, base, ldc)[1]
        assert want in plan and "last round" not in plan, plan
        rc, out = run(dtype, M, N, K, 1.5, A, lda, B, ldb, -0.75, C, ldc, "chosen " + want)
    assert rc == 0
    check(dtype, M, N, K, 1.5, A, lda, B, ldb, -0.75, C, ldc, out, "chosen %s %s" % (dtype, want))


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_k_deterministic_and_paths_agree(dtype):
    """A split call gives the same bits twice, with element-wise loads forced
    (same chunking and summation order), and on every tile configuration the
    chunks are reduced in order; its result is within the bound of the
    unsplit one."""
    import dense_gemm_fp32_amd as dg
    t, tc = _t(dtype), _tc(dtype)
    M, N, K = 333, 456, 1500
    rng = np.random.default_rng(8)
    A = rng.standard_normal(M * K).astype(t)
    B = rng.standard_normal(K * N).astype(t)
    C = rng.standard_normal(M * N).astype(tc)
    with split_mode(5):
        rc1, o1 = run(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, "split det1")
        rc2, o2 = run(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, "split det2")
        prev = dg.gemm_set_load_mode(1)
        try:
            rc3, o3 = run(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, "split scalar")
        finally:
            dg.gemm_set_load_mode(prev)
    assert rc1 == rc2 == rc3 == 0
    assert np.array_equal(bits(o1, dtype), bits(o2, dtype))
    assert np.array_equal(bits(o1, dtype), bits(o3, dtype))
    check(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, o1, "split det")
    for cfg in (1, 2, 3, 4, 6, 9, 10):
        with split_mode(3), tile_config(cfg):
            rc, o = run(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, "split cfg%d" % cfg)
        assert rc == 0
        check(dtype, M, N, K, 0.5, A, K, B, N, 2.0, C, N, o, "split 3 cfg %d" % cfg)


@pytest.mark.parametrize("dtype,M,N,K", [("f32", 2304, 2304, 5000), ("f16", 1024, 1024, 8192),
                                          ("f16f32", 512, 512, 8192), ("f32", 512, 512, 8192)])
def test_split_k_chosen_by_size_sampled(dtype, M, N, K):
    """Shapes whose tile grid leaves CUs idle take split K by themselves;
    checked on sampled rows, the checksum and Freivalds' product check."""
    import dense_gemm_fp32_amd as dg
    w = wl.Workload("auto_split_%s_%dx%dx%d" % (dtype, M, N, K), dtype, M, N, K, K, N, N, 1.5, -0.5,
                    "uniform", "uniform", (31, 32, 33))
    A, B, C = wl.make(w)
    assert "split-K" in dg.gemm_describe(dtype, M, N, K, w.alpha, A.ctypes.data, K, B.ctypes.data, N,
                                         w.beta, C.ctypes.data, N)[1]
    rc, out = run(dtype, M, N, K, w.alpha, A, K, B, N, w.beta, C, N, w.name)
    assert rc == 0
    check_sampled(dtype, w, A, B, C, out, nrows=32)


def test_split_k_more_chunks_than_k_steps():
    """K = 40 has two 32-wide K steps: a forced split of 7 runs as 2 chunks
    (fp32 tiny tile, K step 32), still matching the oracle."""
    import dense_gemm_fp32_amd as dg
    M, N, K = 96, 80, 40
    rng = np.random.default_rng(9)
    A = rng.uniform(-1, 1, M * K).astype(np.float32)
    B = rng.uniform(-1, 1, K * N).astype(np.float32)
    C = rng.uniform(-1, 1, M * N).astype(np.float32)
    with split_mode(7), tile_config(4):
        assert "split-K 2" in dg.gemm_describe("f32", M, N, K, 1.0, A.ctypes.data, K, B.ctypes.data, N,
                                              1.0, C.ctypes.data, N)[1]
        rc, out = run("f32", M, N, K, 1.0, A, K, B, N, 1.0, C, N, "split7 K40")
    assert rc == 0
    check("f32", M, N, K, 1.0, A, K, B, N, 1.0, C, N, out, "split7 K40")


# ---------------------------------------------------------------- column-major calls

COLMAJOR_SHAPES = [
    # M,   N,   K,  lda, ldb, ldc   (lda >= M, ldb >= K, ldc >= M)
    (300, 200, 100, 300, 100, 300),
    (257, 530, 77, 261, 80, 259),
    (1000, 64, 1500, 1000, 1504, 1008),   # deep K: takes split K in fp32
]


@pytest.mark.parametrize("dtype", DTYPES)
def test_colmajor_matches_oracle(dtype):
    """Column-major operands laid out explicitly (element (i, j) at
    X[i + j*ld]), checked against the oracle on row-major copies of the same
    logical matrices; the pad rows of C's columns must be left unchanged."""
    t, tc = _t(dtype), _tc(dtype)
    for idx, (M, N, K, lda, ldb, ldc) in enumerate(COLMAJOR_SHAPES):
        rng = np.random.default_rng(M + 7 * N + 3 * K)
        A = rng.uniform(-1, 1, (M, K)).astype(t)
        B = rng.uniform(-1, 1, (K, N)).astype(t)
        C = rng.uniform(-1, 1, (M, N)).astype(tc)
        beta = [0.5, 0.0, -1.0][idx % 3]
        Cbuf = colmajor_buf(C, ldc, wl.C_PAD_SENTINEL)
        rc, out = run_colmajor(dtype, M, N, K, 1.5, colmajor_buf(A, lda, np.nan), lda,
                               colmajor_buf(B, ldb, np.nan), ldb, beta, Cbuf, ldc, "colmajor")
        assert rc == 0
        got = colmajor_view(out, M, N, ldc)
        R, G = oracle.gemm(M, N, K, 1.5, np.ascontiguousarray(A).reshape(-1), K,
                           np.ascontiguousarray(B).reshape(-1), N, beta,
                           np.ascontiguousarray(C).reshape(-1) if beta != 0 else None, N, dtype)
        tol = oracle.tolerance(G, np.abs(C.astype(np.float64)) if beta != 0 else 0.0, 1.5, beta, K, R,
                               oracle.out_type(dtype))
        ok, worst, where = oracle.compare(got, R, tol)
        assert ok, "colmajor %s %s: worst %.3g at %s" % (dtype, (M, N, K), worst, where)
        u = np.uint16 if dtype == "f16" else np.uint32
        pads_in = Cbuf.reshape(N, ldc)[:, M:].view(u)
        pads_out = np.asarray(out).reshape(N, ldc)[:, M:].view(u)
        assert np.array_equal(pads_in, pads_out), "pad rows of C were modified"


# ---------------------------------------------------------------- vector-ALU fp32 (ablation)

def test_valu_tails_and_ragged_match_oracle():
    """gemm_f32_valu (the SIMT register-blocked design on the vector ALUs):
    tile-crossing shapes with aligned and unaligned leading dimensions, and
    the ragged workload with NaN pads and a C-pad sentinel."""
    rng = np.random.default_rng(41)
    for idx, (M, N, K) in enumerate([(1, 1, 1), (7, 130, 33), (129, 127, 17), (255, 257, 100),
                                     (300, 200, 1000), (64, 64, 16)]):
        pad = idx % 3
        lda, ldb, ldc = K + 4 * pad, N + pad, N + 2 * pad
        beta = [0.0, 1.0, -0.5][idx % 3]
        A = wl.pad(rng.uniform(-1, 1, (M, K)).astype(np.float32), lda, np.nan)
        B = wl.pad(rng.uniform(-1, 1, (K, N)).astype(np.float32), ldb, np.nan)
        C = wl.pad(rng.uniform(-1, 1, (M, N)).astype(np.float32), ldc, wl.C_PAD_SENTINEL)
        rc, out = run("f32", M, N, K, 1.25, A, lda, B, ldb, beta, C, ldc, "valu", entry="gemm_f32_valu")
        assert rc == 0
        check("f32", M, N, K, 1.25, A, lda, B, ldb, beta, C, ldc, out, "valu %s" % ((M, N, K),))
    w = wl.RAGGED_F32
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, "valu ragged",
                  entry="gemm_f32_valu")
    assert rc == 0
    check(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, out, "valu ragged")


def test_valu_exact_specials_and_deterministic():
    """Small integers (exact in fp32: bitwise equal to the rounded oracle),
    beta = 0 with NaN C, alpha = 0 with NaN A and B, and two identical calls
    giving identical bits."""
    M, N, K = 300, 260, 1000
    A = wl.small_ints(M, K, -8, 8, 1, "f32").reshape(-1)
    B = wl.small_ints(K, N, -8, 8, 2, "f32").reshape(-1)
    C = wl.small_ints(M, N, -8, 8, 3, "f32").reshape(-1)
    rc, out = run("f32", M, N, K, -1.0, A, K, B, N, 2.0, C, N, "valu ints", entry="gemm_f32_valu")
    assert rc == 0
    R, _ = oracle.gemm(M, N, K, -1.0, A, K, B, N, 2.0, C, N)
    assert np.array_equal(bits(out, "f32"), bits(exact_expected("f32", R).reshape(-1), "f32"))
    Cn = np.full(M * N, np.nan, np.float32)
    rc, out = run("f32", M, N, K, 1.0, A, K, B, N, 0.0, Cn, N, "valu beta0", entry="gemm_f32_valu")
    assert rc == 0 and np.all(np.isfinite(out))
    An = np.full(M * K, np.nan, np.float32)
    rc, out = run("f32", M, N, K, 0.0, An, K, An[:K * N], N, 0.5, C, N, "valu alpha0",
                  entry="gemm_f32_valu")
    assert rc == 0 and np.array_equal(out, (np.float32(0.5) * C).astype(np.float32))
    rng = np.random.default_rng(3)
    A = rng.standard_normal(M * K).astype(np.float32)
    rc1, o1 = run("f32", M, N, K, 1.0, A, K, B, N, 1.0, C, N, "valu det1", entry="gemm_f32_valu")
    rc2, o2 = run("f32", M, N, K, 1.0, A, K, B, N, 1.0, C, N, "valu det2", entry="gemm_f32_valu")
    assert rc1 == rc2 == 0 and np.array_equal(bits(o1, "f32"), bits(o2, "f32"))


def test_valu_4096_sampled():
    w = wl.F32_4096
    A, B, C = wl.make(w)
    rc, out = run(w.dtype, w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, "valu 4096",
                  entry="gemm_f32_valu")
    assert rc == 0
    check_sampled(w.dtype, w, A, B, C, out, nrows=24)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [0, 1])
def test_mfma_probe_runs_and_counts(dtype):
    """The matrix-core ceiling probe: its flop count follows its definition
    (512 workgroups x 8 waves x iters x a 128 x 64 wave tile over k, 2*128*64*k
    flops, k = 32 for fp16 and 2 for fp32) and every
    thread's accumulator sum equals iters times the sum after one round (the
    rounds repeat the same products; small integer operands keep every sum
    exact)."""
    import torch
    import dense_gemm_fp32_amd as dg
    from gemm_harness import note
    note("mfma probe dtype=%d" % dtype)
    dev = torch.device("cuda:0")
    tdt = torch.float16 if dtype == 1 else torch.float32
    nvals = 65536 // (2 if dtype == 1 else 4)
    g = torch.Generator().manual_seed(11)
    ops = torch.randint(-2, 3, (nvals,), generator=g).to(tdt).to(dev)
    out1 = torch.empty(512 * 512, dtype=torch.float32, device=dev)
    out3 = torch.empty_like(out1)
    rc, f1 = dg.gemm_probe_mfma(dtype, 1, ops, out1)
    assert rc == 0, dg.gemm_status_string(rc)
    rc, f3 = dg.gemm_probe_mfma(dtype, 3, ops, out3)
    assert rc == 0, dg.gemm_status_string(rc)
    torch.cuda.synchronize(dev)
    k = 32 if dtype == 1 else 2
    assert f1 == 512 * 8 * 1 * 2 * 128 * 64 * k and f3 == 3 * f1
    a1, a3 = out1.cpu().double(), out3.cpu().double()
    assert torch.isfinite(a1).all() and torch.isfinite(a3).all()
    assert torch.equal(a3, 3 * a1)


# ---------------------------------------------------------------- transposed operands

LAYOUTS = ["nt", "tn", "tt"]

# (M, N, K, pad_a, pad_b, pad_c): row lengths as stored plus the pads.  Pads
# of 0 or multiples of 8 keep every row 16-byte aligned (direct loads); odd
# pads force the register-staged path.
LAYOUT_SHAPES = [
    (1000, 3000, 517, 13, 5, 3),       # the ragged workload's sizes, unaligned
    (515, 263, 300, 0, 0, 0),          # tails in M, N and K, aligned
    (296, 200, 160, 8, 16, 4),         # M, N multiples of 8, padded rows
    (256, 512, 384, 0, 0, 0),          # whole tiles
    (33, 17, 1, 0, 0, 0),              # K = 1
    (7, 130, 45, 1, 0, 2),
]


def _layout_run_check(dtype, layout, M, N, K, pads, seed, alpha=1.5, beta=-0.75, label=""):
    from gemm_harness import check_layout, layout_case, run_layout
    ta, tb = layout[0] == "t", layout[1] == "t"
    lda = (M if ta else K) + pads[0]
    ldb = (K if tb else N) + pads[1]
    ldc = N + pads[2]
    Abuf, Bbuf, Cbuf, A, B, C = layout_case(dtype, M, N, K, ta, tb, lda, ldb, ldc, seed)
    rc, out = run_layout(dtype, layout, M, N, K, alpha, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc,
                         label)
    assert rc == 0, rc
    return check_layout(dtype, M, N, K, alpha, A, B, beta, C, Cbuf, ldc, out,
                        "%s %s %s %s" % (label, dtype, layout, (M, N, K)))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_layouts_match_oracle(dtype, layout):
    """gemm_*_nt / _tn / _tt: operands stored transposed (NaN pads, never
    read), every tail and both the direct and the register-staged paths,
    against the oracle on the logical matrices."""
    for idx, (M, N, K, *pads) in enumerate(LAYOUT_SHAPES):
        beta = [-0.75, 0.0, 1.0, 0.5][idx % 4]
        _layout_run_check(dtype, layout, M, N, K, pads, 100 + idx, beta=beta, label="layout")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 6, 7, 8, 9, 10])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_layouts_every_tile(dtype, layout, cfg):
    """Each tile configuration with transposed operands, on a shape with
    edge tiles in M and N (multiples of 8: direct loads up to the edge) and
    one with odd edges (staged loads at the edge)."""
    with tile_config(cfg):
        _layout_run_check(dtype, layout, 296, 200, 160, (0, 0, 0), 200 + cfg, label="cfg%d" % cfg)
        _layout_run_check(dtype, layout, 301, 203, 97, (0, 0, 0), 300 + cfg, beta=0.0,
                          label="cfg%d" % cfg)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_layouts_split_k(dtype, layout):
    """Split K with transposed operands: each chunk's operand offsets follow
    the stored orientation."""
    with split_mode(3):
        _layout_run_check(dtype, layout, 200, 136, 1000, (0, 0, 0), 400, label="split3")
        _layout_run_check(dtype, layout, 129, 77, 515, (3, 1, 2), 401, label="split3 ragged")


@pytest.mark.parametrize("cfg", [1, 6])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_layouts_large_sampled(dtype, layout, cfg):
    """2048^3 with transposed operands on each large tile, forced: fp32 256x128
    (cfg 1) and 256x256 (cfg 6); fp16 256x256 on 16x16x32 blocks (cfg 1; with
    both operands transposed that tile keeps 32x32x16 blocks) and on 32x32x16
    blocks (cfg 6).  32 k-steps of the direct-load pipeline; sampled rows
    against the oracle."""
    from gemm_harness import layout_case, run_layout
    n = 2048
    ta, tb = layout[0] == "t", layout[1] == "t"
    Abuf, Bbuf, Cbuf, A, B, C = layout_case(dtype, n, n, n, ta, tb, n, n, n, 500)
    with tile_config(cfg):
        rc, out = run_layout(dtype, layout, n, n, n, 1.0, Abuf, n, Bbuf, n, 0.5, Cbuf, n,
                             "large cfg%d" % cfg)
    assert rc == 0
    rows = wl.sample_rows(n, 32, 7)
    R, G = oracle.gemm(len(rows), n, n, 1.0, np.ascontiguousarray(A[rows]).reshape(-1), n,
                       B.reshape(-1), n, 0.5, np.ascontiguousarray(C[rows]).reshape(-1), n, dtype)
    tol = oracle.tolerance(G, np.abs(C[rows].astype(np.float64)), 1.0, 0.5, n, R,
                           oracle.out_type(dtype))
    got = wl.view(out, n, n, n)[rows]
    ok, worst, where = oracle.compare(np.ascontiguousarray(got), R, tol)
    assert ok, "%s %s cfg %d 2048^3 sampled: worst %.3g at %s" % (dtype, layout, cfg, worst, where)


def test_tensor_wrapper_takes_transposed_views():
    """dense_gemm_fp32_amd.gemm on X.t() views runs the transposed entry
    points; the result is within the fp32 accumulation bound of the float64
    product of the same logical matrices.  A view with neither rows nor
    columns contiguous is refused."""
    import torch
    import dense_gemm_fp32_amd as dg
    from gemm_harness import note
    note("tensor wrapper transposed views")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(5)
    At = (torch.rand(96, 130, generator=g) * 2 - 1).to(dev)      # stored K x M
    Bt = (torch.rand(70, 96, generator=g) * 2 - 1).to(dev)       # stored N x K
    C = torch.zeros(130, 70, device=dev)
    dg.gemm(At.t(), Bt.t(), C, 1.0, 0.0)
    torch.cuda.synchronize()
    A = At.t().contiguous().cpu().double().numpy()
    B = Bt.t().contiguous().cpu().double().numpy()
    R = A @ B
    bound = 4 * 96 * 2.0 ** -24 * (np.abs(A) @ np.abs(B)) + 2.0 ** -24 * np.abs(R) + 1e-30
    assert np.all(np.abs(C.cpu().double().numpy() - R) <= bound)
    with pytest.raises(ValueError):
        dg.gemm(At.t()[::2, ::2], Bt.t()[::2, :], torch.zeros(65, 70, device=dev))


# ---------------------------------------------------------------- split of the last round (fp32)

@contextmanager
def tail_split(mode):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_tail_split(mode)
    try:
        yield
    finally:
        dg.gemm_set_tail_split(prev)


# (tile config, M, N, K): more tiles than CUs, so whole rounds run first and
# the leftover tiles (the last ones of the grouped order) run split.
TAIL_CASES = [
    (1, 4200, 2000, 256),     # 256x128: 17 x 16 = 272 tiles -> 256 + 16
    (2, 2200, 1900, 300),     # 128x128: 18 x 15 = 270 tiles -> 256 + 14
    (3, 1100, 1000, 200),     # 64x64:   18 x 16 = 288 tiles -> 256 + 32
    (4, 600, 600, 700),       # 32x32:   19 x 19 = 361 tiles -> 256 + 105
    (6, 4200, 4200, 256),     # 256x256: 17 x 17 = 289 tiles -> 256 + 33
]


@pytest.mark.parametrize("S", [2, 5])
@pytest.mark.parametrize("case", TAIL_CASES, ids=["big", "mid", "small", "tiny", "huge"])
def test_tail_split_matches_oracle(case, S):
    """The last round's tiles as an S-way split-K pass writing dense tile
    blocks, then the tile reduction (alpha, beta, edges), after the whole
    rounds: every element against the oracle, pads and guard untouched, and
    the same bits on a second call."""
    cfg, M, N, K = case
    from gemm_harness import check_layout, layout_case, run_layout
    for idx, (layout, beta) in enumerate([("nn", 0.5), ("tt", 0.0)]):
        ta, tb = layout[0] == "t", layout[1] == "t"
        lda, ldb, ldc = (M if ta else K), (K if tb else N), N + 4
        Abuf, Bbuf, Cbuf, A, B, C = layout_case("f32", M, N, K, ta, tb, lda, ldb, ldc, 600 + idx)
        with tile_config(cfg), tail_split(S):
            if layout == "nn":
                rc, out = run("f32", M, N, K, 1.25, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc,
                              tag="tail S=%d cfg%d" % (S, cfg))
                rc2, out2 = run("f32", M, N, K, 1.25, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc,
                                tag="tail again")
                assert rc2 == 0 and np.array_equal(bits(out, "f32"), bits(out2, "f32"))
            else:
                rc, out = run_layout("f32", layout, M, N, K, 1.25, Abuf, lda, Bbuf, ldb, beta, Cbuf,
                                     ldc, "tail S=%d cfg%d" % (S, cfg))
        assert rc == 0
        check_layout("f32", M, N, K, 1.25, A, B, beta, C, Cbuf, ldc, out,
                     "tail S=%d cfg%d %s" % (S, cfg, layout))


def test_tail_split_chosen_by_size():
    """A size whose last round the model splits (5504^3 on the 128x128
    tile: 1849 tiles, 7 rounds and 57 left) matches the oracle on sampled
    rows that include the last tile rows (where the leftover tiles of the
    grouped order lie)."""
    import dense_gemm_fp32_amd as dg
    n = 5504
    rc, plan = dg.gemm_describe("f32", n, n, n, 1.0, 0x10000, n, 0x10000, n, 1.0, 0x10000, n)
    assert rc == 0 and "last round split-K" in plan, plan
    from gemm_harness import layout_case
    Abuf, Bbuf, Cbuf, A, B, C = layout_case("f32", n, n, n, False, False, n, n, n, 700)
    rc, out = run("f32", n, n, n, 1.0, Abuf, n, Bbuf, n, 1.0, Cbuf, n, tag="tail by size")
    assert rc == 0
    rows = np.unique(np.concatenate([wl.sample_rows(n, 24, 3), np.arange(n - 40, n)]))
    R, G = oracle.gemm(len(rows), n, n, 1.0, np.ascontiguousarray(A[rows]).reshape(-1), n,
                       B.reshape(-1), n, 1.0, np.ascontiguousarray(C[rows]).reshape(-1), n, "f32")
    tol = oracle.tolerance(G, np.abs(C[rows].astype(np.float64)), 1.0, 1.0, n, R, oracle.out_type("f32"))
    ok, worst, where = oracle.compare(np.ascontiguousarray(wl.view(out, n, n, n)[rows]), R, tol)
    assert ok, "5504^3 last-round split: worst %.3g at %s" % (worst, where)


def test_concurrent_streams_and_threads_share_the_workspace_pool():
    """Split-K calls on two streams, issued from two host threads at once,
    each take their own workspace blocks from the library's pool (requests
    of different sizes, so the pool grows while the other stream holds a
    block): every result equals the same call run alone, bit for bit (the
    chunks are summed in a fixed order)."""
    import threading
    import torch
    import dense_gemm_fp32_amd as dg
    from gemm_harness import note
    note("concurrent streams and threads: split K 8 and 5 by size, last-round split 3")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(21)
    cases = [(512, 520, 4096), (1000, 700, 3000), (4200, 2000, 256)]
    data = []
    for M, N, K in cases:
        A = (torch.rand(M, K, generator=g) * 2 - 1).to(dev)
        B = (torch.rand(K, N, generator=g) * 2 - 1).to(dev)
        data.append((M, N, K, A, B))
    # by size: 128x128 split-K 8, split-K 5; forced: the last round split 3
    with tail_split(3):
        for M, N, K, A, B in data:
            rc, plan = dg.gemm_describe("f32", M, N, K, 1.0, A, K, B, N, 0.0, A, N)
            assert "split-K" in plan, plan
        ref = []
        for M, N, K, A, B in data:
            C = torch.zeros(M, N, device=dev)
            assert dg.gemm_f32(M, N, K, 1.0, A, K, B, N, 0.0, C, N, None) == 0
            torch.cuda.synchronize()
            ref.append(C.clone())
        streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
        outs = [[torch.full((M, N), float("nan"), device=dev) for (M, N, K, A, B) in data]
                for _ in streams]
        torch.cuda.synchronize()
        errors = []

        def worker(t):
            try:
                for rep in range(6):
                    for i, (M, N, K, A, B) in enumerate(data[::(1 if t == 0 else -1)]):
                        j = i if t == 0 else len(data) - 1 - i
                        rc = dg.gemm_f32(M, N, K, 1.0, A, K, B, N, 0.0, outs[t][j], N, streams[t])
                        if rc != 0:
                            errors.append(rc)
            except Exception as e:          # reported below, on the main thread
                errors.append(repr(e))

        threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for t in range(2):
            for j in range(len(data)):
                assert torch.equal(outs[t][j], ref[j]), (t, cases[j])


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(dtype=st.sampled_from(DTYPES), layout=st.sampled_from(LAYOUTS),
       M=st.integers(1, 300), N=st.integers(1, 300), K=st.integers(1, 300),
       pads=st.tuples(st.integers(0, 9), st.integers(0, 9), st.integers(0, 9)),
       beta=st.sampled_from([0.0, 1.0, -1.5]),
       cfg=st.sampled_from([0, 1, 2, 3, 4, 6, 7, 8, 9, 10]),
       split=st.sampled_from([0, 1, 3]),
       pack=st.sampled_from([0, 2]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_layouts_match_oracle(dtype, layout, M, N, K, pads, beta, cfg, split, pack, seed):
    """Random small shapes with transposed operands: random row padding
    (aligned and unaligned), beta, forced tile configurations and splits,
    and operand copies by size or forced."""
    with tile_config(cfg), split_mode(split), pack_mode(pack):
        _layout_run_check(dtype, layout, M, N, K, pads, seed % 100000, beta=beta,
                          label="hyp cfg%d split%d" % (cfg, split))


def test_calls_replay_from_a_captured_graph():
    """Library calls captured into a HIP graph (torch.cuda.CUDAGraph on a
    side stream) -- unsplit fp32 and fp16, a whole split K, a last-round
    split, a Stream-K call, and a call whose unaligned operands are copied to
    16-byte rows, whose workspace becomes an allocation node of the graph --
    replay the eager results bit for bit, several times, with eager GEMMs and
    synchronisations between the replays."""
    import torch
    import dense_gemm_fp32_amd as dg
    from gemm_harness import note
    note("graph capture: unsplit f32/f16, split K 4, last-round split 3, stream-K, operand copies")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(9)
    # (dtype, M, N, K, split mode, tail mode, row pad of A and B)
    cases = [("f32", 1000, 700, 3000, 1, 1, 0), ("f16", 600, 520, 1000, 1, 1, 0),
             ("f32", 1000, 700, 3000, 4, 1, 0), ("f32", 4200, 2000, 256, 1, 3, 0),
             ("f32", 1536, 1536, 1536, 0, 0, 0), ("f32", 2048, 2048, 2048, 0, 0, 1)]
    for dtype, M, N, K, split, tail, pad in cases:
        t = torch.float32 if dtype == "f32" else torch.float16
        fn = dg.gemm_f32 if dtype == "f32" else dg.gemm_f16
        lda, ldb = K + pad, N + pad
        A = (torch.rand(M, lda, generator=g) * 2 - 1).to(t).to(dev)
        B = (torch.rand(K, ldb, generator=g) * 2 - 1).to(t).to(dev)
        C0 = (torch.rand(M, N, generator=g) * 2 - 1).to(t).to(dev)
        plan = dg.gemm_describe(dtype, M, N, K, 1.25, A, lda, B, ldb, 0.5, C0, N)[1]
        assert ("copies A B" in plan) == (pad > 0), plan
        assert ("stream-K" in plan) == (M == 1536), plan
        with split_mode(split), tail_split(tail):
            ref = C0.clone()
            assert fn(M, N, K, 1.25, A, lda, B, ldb, 0.5, ref, N, None) == 0
            torch.cuda.synchronize()
            C = C0.clone()
            s = torch.cuda.Stream(device=dev)
            graph = torch.cuda.CUDAGraph()
            s.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(s):
                graph.capture_begin()
                rc = fn(M, N, K, 1.25, A, lda, B, ldb, 0.5, C, N, s)
                graph.capture_end()
            torch.cuda.synchronize()
            assert rc == 0
            for rep in range(3):
                C.copy_(C0)
                other = torch.zeros(M, N, dtype=t, device=dev)
                assert fn(M, N, K, 1.0, A, lda, B, ldb, 0.0, other, N, None) == 0   # eager work between
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                assert torch.equal(C, ref), (dtype, M, N, K, split, tail, pad, rep)
            del graph


@contextmanager
def workspace_limit(nbytes):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_workspace_limit(nbytes)
    try:
        yield
    finally:
        dg.gemm_set_workspace_limit(prev)


@pytest.mark.parametrize("dtype,M,N,K", [("f32", 2304, 2304, 2304), ("f32", 2944, 2944, 2944),
                                         ("f16", 512, 512, 8192), ("f16f32", 512, 512, 8192)])
def test_workspace_refused_runs_unsplit(dtype, M, N, K):
    """With the workspace limit at 0 every split request fails: the call runs
    unsplit (the fallback the header promises), bitwise equal to the same call
    with splitting switched off, and within the bound of the oracle.  Then a
    limit just below the call's workspace does the same, and a limit at it lets
    the call split again (bitwise equal to the default)."""
    import dense_gemm_fp32_amd as dg
    w = wl.Workload("wslimit_%s_%d" % (dtype, M), dtype, M, N, K, K, N, N, 1.0, 0.5, "uniform",
                    "uniform", (31, 32, 33))
    rc, plan = dg.gemm_describe(dtype, M, N, K, 1.0, 4096, K, 4096, N, 0.5, 4096, N)
    assert rc == 0 and "workspace" in plan, plan
    nbytes = int(plan.split("workspace ")[1].split()[0])
    A, B, C = wl.make(w)
    with workspace_limit(0):
        rc, out0 = run(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, "limit 0 (%s)" % plan)
    assert rc == 0
    with workspace_limit(nbytes - 1):
        rc, out1 = run(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, "limit below")
    assert rc == 0
    with split_mode(1), tail_split(1):
        rc, ref = run(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, "unsplit")
    assert rc == 0
    assert np.array_equal(bits(out0, dtype), bits(ref, dtype))
    assert np.array_equal(bits(out1, dtype), bits(ref, dtype))
    check(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, out0, "workspace refused")
    with workspace_limit(nbytes):
        rc, out2 = run(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, "limit at")
    assert rc == 0
    rc, dflt = run(dtype, M, N, K, 1.0, A, K, B, N, 0.5, C, N, "default")
    assert rc == 0
    assert np.array_equal(bits(out2, dtype), bits(dflt, dtype))


# ---------------------------------------------------------------- operand copies

@contextmanager
def pack_mode(mode):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_pack(mode)
    assert prev in (0, 1, 2)
    try:
        yield
    finally:
        dg.gemm_set_pack(prev)


def _layout_outputs(dtype, layout, M, N, K, pads, seed, alpha, beta, label):
    """Stored operands (NaN pads) of a call in `layout` ("nn" = gemm_<dtype>)
    and the call's output; returns (A, B, C, Cbuf, ldc, out)."""
    from gemm_harness import layout_case, run_layout
    ta, tb = layout[0] == "t", layout[1] == "t"
    lda = (M if ta else K) + pads[0]
    ldb = (K if tb else N) + pads[1]
    ldc = N + pads[2]
    Abuf, Bbuf, Cbuf, A, B, C = layout_case(dtype, M, N, K, ta, tb, lda, ldb, ldc, seed)
    if layout == "nn":
        rc, out = run(dtype, M, N, K, alpha, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc, label)
    else:
        rc, out = run_layout(dtype, layout, M, N, K, alpha, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc,
                             label)
    assert rc == 0, rc
    return A, B, C, Cbuf, ldc, out


# (M, N, K, pad_a, pad_b, pad_c): odd pads leave the rows of that operand
# without 16-byte alignment, so it is copied when copies are forced.
COPY_SHAPES = [
    (1000, 3000, 517, 13, 5, 3),       # the ragged workload's sizes: A and B copied
    (301, 203, 97, 1, 3, 0),           # tails in M, N and K
    (256, 512, 384, 1, 0, 0),          # only A copied
    (256, 512, 384, 0, 1, 8),          # only B copied
    (7, 130, 45, 1, 0, 2),
]


@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_operand_copies_match_oracle_and_staged_path(dtype, layout):
    """Copies forced (gemm_set_pack(2)) against copies off (1), under the same
    forced tile and split: the copy is bit-exact and the kernels sum the same
    products in the same order, so the outputs are the same bits; both within
    the oracle's bound, NaN pads never read (the copy reads only the matrix
    and writes zeros into its own pads)."""
    from gemm_harness import check_layout
    for idx, (M, N, K, *pads) in enumerate(COPY_SHAPES):
        beta = [-0.75, 0.0, 1.0, 0.5, 0.25][idx]
        outs = []
        for mode in (2, 1):
            with pack_mode(mode), tile_config(2), split_mode(1):
                A, B, C, Cbuf, ldc, out = _layout_outputs(dtype, layout, M, N, K, pads, 700 + idx,
                                                          1.5, beta, "pack%d" % mode)
            check_layout(dtype, M, N, K, 1.5, A, B, beta, C, Cbuf, ldc, out,
                         "pack %d %s" % (mode, (M, N, K)))
            outs.append(out)
        assert np.array_equal(bits(outs[0], dtype), bits(outs[1], dtype)), (dtype, layout, M, N, K)
        # and with the tile and split the rule picks for the copies
        with pack_mode(2):
            A, B, C, Cbuf, ldc, out = _layout_outputs(dtype, layout, M, N, K, pads, 700 + idx, 1.5,
                                                      beta, "pack2 by size")
        check_layout(dtype, M, N, K, 1.5, A, B, beta, C, Cbuf, ldc, out, "pack 2 by size")


@pytest.mark.parametrize("dtype", DTYPES)
def test_operand_copy_of_a_misaligned_base(dtype):
    """Leading dimensions that allow 16-byte rows, but A and B start one
    element past a 16-byte boundary: the rows are copied (forced) to an
    aligned buffer; bitwise equal to the staged path under the same tile and
    split, and within the oracle's bound."""
    import torch
    import dense_gemm_fp32_amd as dg
    M, N, K = 384, 320, 256
    rng = np.random.default_rng(91)
    t = _t(dtype)
    A = rng.uniform(-1, 1, (M, K)).astype(t)
    B = rng.uniform(-1, 1, (K, N)).astype(t)
    C = rng.uniform(-1, 1, (M, N)).astype(_tc(dtype))
    dev = torch.device("cuda:0")
    fn = {"f32": dg.gemm_f32, "f16": dg.gemm_f16, "f16f32": dg.gemm_f16f32}[dtype]
    outs = []
    for mode in (2, 1):
        note("misaligned base, copies mode %d, %s %dx%dx%d" % (mode, dtype, M, N, K))
        # one leading element, so the matrices start 4 (fp32) or 2 (fp16) bytes in
        dA = torch.from_numpy(np.concatenate([np.zeros(1, t), A.reshape(-1)])).to(dev)
        dB = torch.from_numpy(np.concatenate([np.zeros(1, t), B.reshape(-1)])).to(dev)
        dC = torch.from_numpy(C.reshape(-1).copy()).to(dev)
        with pack_mode(mode), tile_config(2), split_mode(1):
            rc, plan = dg.gemm_describe(dtype, M, N, K, 1.0, dA[1:], K, dB[1:], N, 0.5, dC, N)
            assert rc == 0 and (("copies A B" in plan) == (mode == 2)), plan
            rc = fn(M, N, K, 1.0, dA[1:], K, dB[1:], N, 0.5, dC, N,
                    torch.cuda.current_stream(dev))
        torch.cuda.synchronize(dev)
        assert rc == 0
        outs.append(dC.cpu().numpy())
    assert np.array_equal(bits(outs[0], dtype), bits(outs[1], dtype))
    check(dtype, M, N, K, 1.0, A.reshape(-1), K, B.reshape(-1), N, 0.5, C.reshape(-1), N, outs[0],
          "misaligned base copied")


@pytest.mark.parametrize("dtype", ["f32", "f16", "f16f32"])
def test_operand_copies_chosen_by_size_sampled(dtype):
    """2048^3 with every leading dimension 2049: above the fp32 size rule, so
    A and B are copied and the GEMM runs the direct-load kernels on the
    copies (fp16 copies forced: no size rule copies them); sampled rows
    against the oracle, plus the last tile row and column."""
    if dtype == "f32":
        _copies_2048(dtype)
    else:
        with pack_mode(2):
            _copies_2048(dtype)


def _copies_2048(dtype):
    import dense_gemm_fp32_amd as dg
    n = 2048
    w = wl.Workload("copies_%s_%d" % (dtype, n), dtype, n, n, n, n + 1, n + 1, n + 1, 1.0, 0.5,
                    "uniform", "uniform", (61, 62, 63))
    rc, plan = dg.gemm_describe(dtype, n, n, n, 1.0, 4096, n + 1, 4096, n + 1, 0.5, 4096, n + 1)
    assert rc == 0 and "copies A B" in plan, plan
    A, B, C = wl.make(w)
    rc, out = run(dtype, n, n, n, 1.0, A, n + 1, B, n + 1, 0.5, C, n + 1, "copies by size (%s)" % plan)
    assert rc == 0
    check_sampled(dtype, w, A, B, C, out, nrows=24, seed=11, extra_rows=[n - 1, n - 129])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_operand_copies_refused_fall_back(dtype):
    """With no workspace to be had (limit 0) a call that would copy its
    operands (fp32 above the size rule; fp16 with copies forced) runs on its
    original operands, unsplit: bitwise equal to copies and splitting switched
    off, within the oracle's bound."""
    n = 2048
    w = wl.Workload("copies_refused_%s" % dtype, dtype, n, n, n, n + 1, n + 1, n + 1, 1.0, 0.5,
                    "uniform", "uniform", (64, 65, 66))
    A, B, C = wl.make(w)
    with workspace_limit(0), pack_mode(0 if dtype == "f32" else 2):
        rc, out0 = run(dtype, n, n, n, 1.0, A, n + 1, B, n + 1, 0.5, C, n + 1, "copies refused")
    assert rc == 0
    with pack_mode(1), split_mode(1), tail_split(1):
        rc, ref = run(dtype, n, n, n, 1.0, A, n + 1, B, n + 1, 0.5, C, n + 1, "no copies, unsplit")
    assert rc == 0
    assert np.array_equal(bits(out0, dtype), bits(ref, dtype))
    check_sampled(dtype, w, A, B, C, out0, nrows=12, seed=12)


# ---------------------------------------------------------------- Stream-K

@contextmanager
def stream_k(mode):
    import dense_gemm_fp32_amd as dg
    prev = dg.gemm_set_stream_k(mode)
    assert 0 <= prev <= 6
    try:
        yield
    finally:
        dg.gemm_set_stream_k(prev)


# (M, N, K, pad_a, pad_b, pad_c, beta) on the 64x64 tile, every Stream-K mode
STREAMK_CASES = [
    (1100, 1200, 1300, 0, 0, 0, 0.5),   # 342 tiles; tails in M, N and K
    (1152, 1152, 1152, 0, 0, 3, 1.0),   # C rows not 16-byte aligned: element-wise fix-up
    (700, 1900, 333, 0, 0, 0, 0.0),     # beta 0 over a NaN C; K rows without 16-byte loads
    (1090, 1500, 64, 4, 0, 0, -0.75),   # two K steps: runs shorter than a tile, many shared tiles
]


@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
def test_stream_k_every_mode_matches_oracle(layout):
    """Every Stream-K decomposition of the 64x64 tile (every tile's K steps
    over 1, 2 or 3 workgroups per CU; whole rounds first, the rest over 1 or
    2 more per CU) and the plain launch, in each layout, against the oracle
    element by element: shared tiles summed from their parts, tiles a run
    covers whole written directly, ragged edges, alpha and beta applied once,
    C pads untouched, and with beta = 0 a C full of NaN never read.  A second
    call of each mode gives the same bits (the fix-up sums parts in K order)."""
    import dense_gemm_fp32_amd as dg
    from gemm_harness import layout_case, run_layout
    ta, tb = layout[0] == "t", layout[1] == "t"
    for idx, (M, N, K, pa, pb, pc, beta) in enumerate(STREAMK_CASES):
        lda = (M if ta else K) + pa
        ldb = (K if tb else N) + pb
        ldc = N + pc
        Abuf, Bbuf, Cbuf, A, B, C = layout_case("f32", M, N, K, ta, tb, lda, ldb, ldc, 900 + idx)
        if beta == 0.0:
            Cbuf = wl.pad(np.full((M, N), np.nan, np.float32), ldc, wl.C_PAD_SENTINEL)
        R, G = oracle.gemm(M, N, K, 1.5, A.reshape(-1), K, B.reshape(-1), N, beta,
                           np.ascontiguousarray(C).reshape(-1) if beta != 0 else None, N, "f32")
        Cv = C.astype(np.float64) if beta != 0 else 0.0
        tol = oracle.tolerance(G, np.abs(Cv), 1.5, beta, K, R, oracle.out_type("f32"))
        for mode in (1, 2, 3, 4, 5, 6):
            label = "stream-K mode %d %s %dx%dx%d" % (mode, layout, M, N, K)
            with stream_k(mode), tile_config(7):
                # (gemm_describe takes the untransposed layout; the forced
                # mode decides Stream-K whatever the layout)
                rc, plan = dg.gemm_describe("f32", M, N, K, 1.5, 4096, K + pa, 4096, N + pb, beta,
                                            4096, ldc)
                assert rc == 0 and ("stream-K" in plan) == (mode >= 2), plan
                outs = []
                for rep in range(2):
                    if layout == "nn":
                        rc, out = run("f32", M, N, K, 1.5, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc,
                                      label)
                    else:
                        rc, out = run_layout("f32", layout, M, N, K, 1.5, Abuf, lda, Bbuf, ldb,
                                             beta, Cbuf, ldc, label)
                    assert rc == 0, rc
                    outs.append(out)
            assert np.array_equal(bits(outs[0], "f32"), bits(outs[1], "f32")), label
            gpu = wl.view(outs[0], M, N, ldc)
            ok, worst, where = oracle.compare(gpu, R, tol)
            assert ok, "%s (%s): worst |err|/tol %.3g at %s" % (label, plan, worst, where)
            assert_pads_unchanged(outs[0], Cbuf, M, N, ldc, "f32")


# tile configuration -> (M, N, K, pad_a, pad_b, pad_c, beta) cases: one grid
# over a round of that tile's tiles (whole tiles first in modes 5, 6), one
# under it
STREAMK_TILE_CASES = {
    6: [(4300, 4400, 333, 0, 0, 0, 0.5), (900, 1300, 515, 0, 0, 1, 0.0)],   # 256x256
    1: [(4300, 2200, 700, 0, 4, 0, -0.75), (1500, 700, 260, 0, 0, 0, 1.0)],  # 256x128
    5: [(2200, 2200, 1000, 0, 0, 3, 0.0), (900, 1300, 515, 4, 0, 0, 0.5)],   # 128x128
    8: [(2200, 2250, 1100, 0, 4, 1, 0.5), (700, 1500, 515, 0, 0, 0, 0.0)],   # 128x64
}


@pytest.mark.parametrize("layout", ["nn", "nt", "tn", "tt"])
@pytest.mark.parametrize("cfg", [6, 1, 5, 8], ids=["256x256", "256x128", "128x128", "128x64"])
def test_stream_k_large_tiles_every_mode_matches_oracle(cfg, layout):
    """Stream-K on the 256x256, 256x128, 128x128 and 128x64 tiles, in every mode
    and layout, against the oracle element by element: runs of one K step up
    to a whole tile, partial K steps, ragged edges, C rows not 16-byte
    aligned, beta = 0 over a NaN C, pads untouched."""
    import dense_gemm_fp32_amd as dg
    from gemm_harness import layout_case, run_layout
    ta, tb = layout[0] == "t", layout[1] == "t"
    for idx, (M, N, K, pa, pb, pc, beta) in enumerate(STREAMK_TILE_CASES[cfg]):
        lda = (M if ta else K) + pa
        ldb = (K if tb else N) + pb
        ldc = N + pc
        Abuf, Bbuf, Cbuf, A, B, C = layout_case("f32", M, N, K, ta, tb, lda, ldb, ldc,
                                                 950 + 10 * cfg + idx)
        if beta == 0.0:
            Cbuf = wl.pad(np.full((M, N), np.nan, np.float32), ldc, wl.C_PAD_SENTINEL)
        R, G = oracle.gemm(M, N, K, 1.25, A.reshape(-1), K, B.reshape(-1), N, beta,
                           np.ascontiguousarray(C).reshape(-1) if beta != 0 else None, N, "f32")
        Cv = C.astype(np.float64) if beta != 0 else 0.0
        tol = oracle.tolerance(G, np.abs(Cv), 1.25, beta, K, R, oracle.out_type("f32"))
        for mode in (2, 3, 4, 5, 6):
            label = "stream-K cfg %d mode %d %s %dx%dx%d" % (cfg, mode, layout, M, N, K)
            with stream_k(mode), tile_config(cfg):
                rc, plan = dg.gemm_describe("f32", M, N, K, 1.25, 4096, K + pa, 4096, N + pb, beta,
                                            4096, ldc)
                assert rc == 0 and "stream-K" in plan, plan
                if layout == "nn":
                    rc, out = run("f32", M, N, K, 1.25, Abuf, lda, Bbuf, ldb, beta, Cbuf, ldc, label)
                else:
                    rc, out = run_layout("f32", layout, M, N, K, 1.25, Abuf, lda, Bbuf, ldb, beta,
                                         Cbuf, ldc, label)
            assert rc == 0, rc
            ok, worst, where = oracle.compare(wl.view(out, M, N, ldc), R, tol)
            assert ok, "%s (%s): worst |err|/tol %.3g at %s" % (label, plan, worst, where)
            assert_pads_unchanged(out, Cbuf, M, N, ldc, "f32")


def test_stream_k_128x128_chosen_by_size_full_oracle():
    """3840^3 (beta = 1), where the size rule runs 768 128x128 tiles whole and
    the last 132 tiles' K steps Stream-K, against the full oracle."""
    w = wl.sweep(3840)
    plan = _plan(w)
    assert "128x128x16" in plan and "stream-K after 768 whole tiles" in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("shape", [(2176, 2176, 2176), (2560, 2560, 2560), (2688, 2688, 2688),
                                   (2048, 2304, 2048), (2200, 2300, 1500), (768, 6144, 2048),
                                   (900, 5000, 700)])
def test_stream_k_128x64_tile_chosen_by_size_full_oracle(shape):
    """Calls (beta = 1) with two to three and a half rounds of 128x64 tiles,
    the last partly filled (2176^3: 578 tiles; 2560^3: 800; 2688^3: 882;
    2048 x 2304 x 2048: 576; 2200 x 2300 x 1500: 648, ragged in M and N;
    768 x 6144 x 2048: 576, narrow; 900 x 5000 x 700: 632, ragged and short):
    the whole rounds run whole and the leftover tiles' K steps Stream-K on
    the same tile; every element against the oracle."""
    M, N, K = shape
    w = wl.sweep(M) if M == N == K else wl.Workload(
        "streamk_%dx%dx%d" % shape, "f32", M, N, K, K, N, N, 1.0, 1.0, "uniform", "uniform",
        (94, 95, 96))
    plan = _plan(w)
    assert "128x64x32 4 waves" in plan and "stream-K after" in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("shape", [(1536, 4096, 1536), (4096, 1536, 2048), (1000, 6144, 1100)])
def test_f32_six_four_wave_tiles_per_cu_full_oracle(shape):
    """Calls (beta = 1) with exactly 1536 64x64 tiles, six on every CU at
    three resident workgroups (1000 x 6144 x 1100 ragged in M and K): the
    four-wave 64x64 tile, plain; every element against the oracle."""
    M, N, K = shape
    w = wl.Workload("six_per_cu_%dx%dx%d" % shape, "f32", M, N, K, K, N, N, 1.0, 1.0, "uniform",
                    "uniform", (97, 98, 99))
    plan = _plan(w)
    assert "64x64x32 4 waves 3 slots" in plan and "stream-K" not in plan, plan
    assert "split" not in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("shape", [(1856, 1856, 1856), (2048, 1600, 1800), (1700, 1900, 1500)])
def test_stream_k_four_wave_tile_past_three_rounds_full_oracle(shape):
    """Calls (beta = 1) with three whole rounds of four-wave 64x64 tiles and at
    most a third of a round more (1856^3: 841 tiles; 2048 x 1600 x 1800: 800;
    1700 x 1900 x 1500: 810, ragged in M and N): the whole rounds run whole and
    the leftover tiles' K steps Stream-K; every element against the oracle."""
    M, N, K = shape
    w = wl.sweep(M) if M == N == K else wl.Workload(
        "streamk_%dx%dx%d" % shape, "f32", M, N, K, K, N, N, 1.0, 1.0, "uniform", "uniform",
        (91, 92, 93))
    plan = _plan(w)
    assert "64x64x32 4 waves" in plan and "stream-K after 768 whole tiles" in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


@pytest.mark.parametrize("shape,tile,whole", [((5632, 5632, 5632), "256x256x32", 256),
                                              ((5120, 3200, 2048), "256x128x32", 256)])
def test_stream_k_large_tiles_chosen_by_size_full_oracle(shape, tile, whole):
    """Calls (beta = 1) whose 256x256 (5632^3: 484 tiles) or 256x128 (5120 x
    3200 x 2048: 500 tiles) tiles leave a round partly filled: the whole
    rounds run whole and the leftover tiles' K steps Stream-K on the same
    tile; every element against the oracle."""
    M, N, K = shape
    w = wl.sweep(M) if M == N == K else wl.Workload(
        "streamk_%dx%dx%d" % shape, "f32", M, N, K, K, N, N, 1.0, 1.0, "uniform", "uniform",
        (81, 82, 83))
    plan = _plan(w)
    assert tile in plan and "stream-K after %d whole tiles" % whole in plan, plan
    _w_run_check(w, "%s (%s)" % (w.name, plan))


def test_stream_k_element_wise_loads_same_bits():
    """Stream-K with the element-wise load switch (register-staged loads, an
    element-wise fix-up) gives the bits of the 16-byte-load run: the same
    products are summed in the same order, whichever way the data moves."""
    import dense_gemm_fp32_amd as dg
    M, N, K = 1536, 1536, 1100
    w = wl.Workload("streamk_loads", "f32", M, N, K, K, N, N, 1.0, 0.25, "uniform", "uniform",
                    (71, 72, 73))
    A, B, C = wl.make(w)
    outs = []
    for scalar in (False, True):
        prev = dg.gemm_set_load_mode(1 if scalar else 0)
        try:
            with stream_k(5):
                rc, plan = dg.gemm_describe("f32", M, N, K, 1.0, 4096, K, 4096, N, 0.25, 4096, N)
                assert "stream-K after 512 whole tiles" in plan, plan
                rc, out = run("f32", M, N, K, 1.0, A, K, B, N, 0.25, C, N,
                              "stream-K loads %s" % ("element-wise" if scalar else "16-byte"))
        finally:
            dg.gemm_set_load_mode(prev)
        assert rc == 0
        outs.append(out)
    assert np.array_equal(bits(outs[0], "f32"), bits(outs[1], "f32"))
    check_sampled("f32", w, A, B, C, outs[0], nrows=16, seed=13, extra_rows=[M - 1, M - 64])


def test_stream_k_refused_falls_back():
    """With the workspace capped below the partial blocks' 8 MiB, a call the
    rule would run Stream-K runs the plain launch: the bits of Stream-K
    switched off."""
    import dense_gemm_fp32_amd as dg
    n = 1536
    w = wl.sweep(n)
    A, B, C = wl.make(w)
    with workspace_limit(1 << 20):
        rc, plan = dg.gemm_describe("f32", n, n, n, w.alpha, 4096, n, 4096, n, w.beta, 4096, n)
        assert rc == 0 and "stream-K" not in plan, plan
        rc, out0 = run("f32", n, n, n, w.alpha, A, n, B, n, w.beta, C, n, "stream-K refused")
    assert rc == 0
    with stream_k(1):
        rc, ref = run("f32", n, n, n, w.alpha, A, n, B, n, w.beta, C, n, "stream-K off")
    assert rc == 0
    assert np.array_equal(bits(out0, "f32"), bits(ref, "f32"))


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(layout=st.sampled_from(["nn"] + LAYOUTS),
       M=st.integers(1, 400), N=st.integers(1, 400), K=st.integers(1, 400),
       pads=st.tuples(st.integers(0, 9), st.integers(0, 9), st.integers(0, 9)),
       beta=st.sampled_from([0.0, 1.0, -1.5]),
       mode=st.sampled_from([2, 3, 4]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_stream_k_match_oracle(layout, M, N, K, pads, beta, mode, seed):
    """Random small shapes on the 64x64 tile with every tile's K steps dealt
    out Stream-K over 1 to 3 workgroups per CU: runs of one K step up to
    several tiles, every tail residue, aligned and unaligned rows, each
    layout."""
    _stream_k_case(layout, M, N, K, pads, beta, mode, seed)


@settings(max_examples=12, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(layout=st.sampled_from(["nn"] + LAYOUTS),
       M=st.integers(1025, 1400), N=st.integers(1025, 1400), K=st.integers(1, 200),
       pads=st.tuples(st.integers(0, 9), st.integers(0, 9), st.integers(0, 9)),
       beta=st.sampled_from([0.0, 1.0, -1.5]),
       mode=st.sampled_from([5, 6]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_stream_k_behind_whole_tiles_match_oracle(layout, M, N, K, pads, beta, mode, seed):
    """Random shapes of 257 to 484 64x64 tiles, short K, with one round of
    whole tiles and the leftover tiles' K steps dealt out to one or two more
    workgroups per CU, each layout, against the oracle."""
    _stream_k_case(layout, M, N, K, pads, beta, mode, seed)


def _stream_k_case(layout, M, N, K, pads, beta, mode, seed):
    from gemm_harness import check_layout
    label = "hyp stream-K mode %d %s %s" % (mode, layout, (M, N, K))
    with tile_config(7), stream_k(mode):
        A, B, C, Cbuf, ldc, out = _layout_outputs("f32", layout, M, N, K, pads, seed % 100000, 1.5,
                                                  beta, label)
    check_layout("f32", M, N, K, 1.5, A, B, beta, C, Cbuf, ldc, out, label)
