"""CPU oracle for row-major C := alpha*A*B + beta*C (fp32; fp16 with fp32
accumulation; fp16 inputs with an fp32 C), evaluated in double precision.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it.

What it computes follows the pages on hand-written GEMM kernels:
  * the SGEMM definition C := alpha*A*B + beta*C with row-major A (M x K),
    B (K x N), C (M x N) and leading dimensions ("Advanced Matrix
    Multiplication on NVIDIA GPUs" summary, opening paragraphs and the section
    on memory layout);
  * C is read only when beta != 0 (same page, tiling section, epilogue);
  * fp16 results are formed in fp32 and rounded once to half with the
    round-to-nearest conversion ("LeetGPU GEMM T4", baseline kernel);
  * the whole-matrix check is the double-precision sum of C ("From 306 ms to
    86 ms", section on how the kernels were timed).

The error bound used by `tolerance` is the one the GEMM's accuracy contract
states: |err| <= 4*K*u*(|alpha|*(|A||B|)_ij + |beta|*|C_ij|) plus the output
rounding step, u = 2^-24 for fp32 accumulation.  Readings of its open points
(K = 0, subnormal outputs, rounding of the perturbed value) are in `tolerance`.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None

U32 = 2.0 ** -24          # unit roundoff of binary32
U16 = 2.0 ** -11          # unit roundoff of binary16
ETA32 = 2.0 ** -149       # smallest positive subnormal binary32
ETA16 = 2.0 ** -24        # smallest positive subnormal binary16


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB_OVERRIDE")   # mutation tests load planted-bug builds
    if not path:
        path = LIB
        if not os.path.exists(LIB):
            build_oracle()
    lib = ctypes.CDLL(path)
    lp = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_gemm_f32.argtypes = [I, I, I, D, lp, L, lp, L, D, lp, L, lp, lp]
    lib.oracle_gemm_f32.restype = I
    lib.oracle_gemm_f16.argtypes = [I, I, I, D, lp, L, lp, L, D, lp, L, lp, lp]
    lib.oracle_gemm_f16.restype = I
    lib.oracle_gemm_f32_elems.argtypes = [I, D, lp, L, lp, L, D, lp, L, L, lp, lp, lp, lp]
    lib.oracle_gemm_f32_elems.restype = None
    lib.oracle_gemm_f16_elems.argtypes = [I, D, lp, L, lp, L, D, lp, L, L, lp, lp, lp, lp]
    lib.oracle_gemm_f16_elems.restype = None
    lib.oracle_gemm_f16f32.argtypes = [I, I, I, D, lp, L, lp, L, D, lp, L, lp, lp]
    lib.oracle_gemm_f16f32.restype = I
    lib.oracle_gemm_f16f32_elems.argtypes = [I, D, lp, L, lp, L, D, lp, L, L, lp, lp, lp, lp]
    lib.oracle_gemm_f16f32_elems.restype = None
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = D
    lib.oracle_double_to_half.argtypes = [D]
    lib.oracle_double_to_half.restype = ctypes.c_uint16
    lib.oracle_double_to_float.argtypes = [D]
    lib.oracle_double_to_float.restype = ctypes.c_float
    lib.oracle_round_to_half.argtypes = [L, lp, lp]
    lib.oracle_round_to_half.restype = None
    lib.oracle_half_to_double_array.argtypes = [L, lp, lp]
    lib.oracle_half_to_double_array.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = I
    _lib = lib
    return lib


def threads():
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_threads())


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _flat(buf, dtype):
    """The caller's padded buffer as a contiguous 1-D array of `dtype`."""
    if buf is None:
        return None
    a = np.ascontiguousarray(buf).reshape(-1)
    if a.dtype != dtype:
        raise TypeError("expected %s buffer, got %s" % (dtype, a.dtype))
    return a


# Storage type of (A and B, C) per call type: "f32" all binary32, "f16" all
# binary16, "f16f32" binary16 inputs with a binary32 C (the output type).
OPERANDS = {"f32": ("f32", "f32"), "f16": ("f16", "f16"), "f16f32": ("f16", "f32")}


def out_type(dtype):
    """Storage type of C and of the result for a call type."""
    return OPERANDS[dtype][1]


def _prep(x, t):
    """Host buffer as a flat array of the storage type t ("f32" / "f16")."""
    if x is None:
        return None
    x = np.asarray(x)
    if t == "f16":
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        return _flat(x, np.uint16)
    return _flat(x, np.float32)


def gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype="f32"):
    """R = alpha*A*B + beta*C in double, and G = |A||B| (both dense M x N).

    A, B, C are host buffers in the library's layout: element (i, j) of a
    matrix with leading dimension ld is buf[i*ld + j].  dtype "f32" takes
    float32 buffers; "f16" takes float16 (or uint16 bit-pattern) buffers.
    "f16f32" takes float16 A and B with a float32 C.  A and B are not read
    when alpha == 0 or K == 0; C is not read when beta == 0 (either may then
    be None).
    """
    lib = _load()
    fns = {"f32": lib.oracle_gemm_f32, "f16": lib.oracle_gemm_f16, "f16f32": lib.oracle_gemm_f16f32}
    if dtype not in fns:
        raise ValueError(dtype)
    fn = fns[dtype]
    tin, tc = OPERANDS[dtype]
    prep = lambda x: _prep(x, tin)
    prep_c = lambda x: _prep(x, tc)

    use_ab = alpha != 0.0 and K > 0
    a = prep(A) if use_ab else None
    b = prep(B) if use_ab else None
    c = prep_c(C) if beta != 0.0 else None
    if use_ab and M > 0 and N > 0:
        _check_span(a, M, K, lda, "A")
        _check_span(b, K, N, ldb, "B")
    if beta != 0.0 and M > 0 and N > 0:
        _check_span(c, M, N, ldc, "C")
    R = np.empty((M, N), np.float64)
    G = np.empty((M, N), np.float64)
    if M > 0 and N > 0:
        rc = fn(M, N, K, float(alpha), _ptr(a), lda, _ptr(b), ldb, float(beta), _ptr(c), ldc,
                _ptr(R), _ptr(G))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
    return R, G


def gemm_elems(rows, cols, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype="f32"):
    """R and G at the listed (rows[t], cols[t]) positions only (1-D arrays)."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be equal-length 1-D arrays")
    fns = {"f32": lib.oracle_gemm_f32_elems, "f16": lib.oracle_gemm_f16_elems,
           "f16f32": lib.oracle_gemm_f16f32_elems}
    if dtype not in fns:
        raise ValueError(dtype)
    fn = fns[dtype]
    tin, tc = OPERANDS[dtype]

    use_ab = alpha != 0.0 and K > 0
    a = _prep(A, tin) if use_ab else None
    b = _prep(B, tin) if use_ab else None
    c = _prep(C, tc) if beta != 0.0 else None
    n = rows.shape[0]
    R = np.empty(n, np.float64)
    G = np.empty(n, np.float64)
    if n:
        fn(K, float(alpha), _ptr(a), lda, _ptr(b), ldb, float(beta), _ptr(c), ldc,
           n, _ptr(rows), _ptr(cols), _ptr(R), _ptr(G))
    return R, G


def _check_span(buf, rows, cols, ld, name):
    if rows <= 0 or cols <= 0:
        return
    need = (rows - 1) * ld + cols
    if buf is None or buf.size < need:
        raise ValueError("%s buffer holds %s elements, needs %d" %
                         (name, None if buf is None else buf.size, need))


# ---- rounding to the output format ----

def round_f16(x):
    """Round float64 values to binary16 (RNE, overflow to +-inf); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    if x.size:
        _load().oracle_round_to_half(x.size, _ptr(x), _ptr(out))
    return out


def half_to_double(bits):
    """Decode binary16 bit patterns (uint16 or float16 arrays) into float64."""
    bits = np.asarray(bits)
    if bits.dtype == np.float16:
        bits = bits.view(np.uint16)
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    if bits.size:
        _load().oracle_half_to_double_array(bits.size, _ptr(bits), _ptr(out))
    return out


def round_f32(x):
    """Round float64 values to binary32 (RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ---- acceptance bound ----

def tolerance(G, Cabs, alpha, beta, K, R, out="f32"):
    """Elementwise bound on |gpu - R| for one GEMM.

        (1 + u_out) * 4 * max(K, 1) * u * (|alpha| G + |beta| |C|)
            + u_out * |R| + eta_out

    u = 2^-24 (fp32 accumulation in both paths).  u_out and eta_out are the
    unit roundoff and the smallest subnormal of the output format: 2^-24 and
    2^-149 for fp32, 2^-11 and 2^-24 for fp16.  Readings of the bound's open
    points: max(K, 1) keeps one rounding for beta*C when K = 0; the factor
    (1 + u_out) covers rounding an already perturbed fp32 value to the output
    format; eta_out covers results in the subnormal range.  Cabs is |C_ij|
    (0 where beta == 0).
    """
    if out == "f32":
        u_out, eta = U32, ETA32
    elif out == "f16":
        u_out, eta = U16, ETA16
    else:
        raise ValueError(out)
    G = np.asarray(G, np.float64)
    Cabs = np.asarray(Cabs, np.float64)
    R = np.asarray(R, np.float64)
    mag = abs(float(alpha)) * G + abs(float(beta)) * Cabs
    return (1.0 + u_out) * 4.0 * max(int(K), 1) * U32 * mag + u_out * np.abs(R) + eta


def compare(gpu, R, tol):
    """Elementwise parity: returns (ok, worst ratio |gpu-R|/tol, index of worst).

    NaN in either side fails unless both are NaN at the same place; infinities
    must match exactly.  gpu is converted to float64 (fp16 via half_to_double).
    """
    gpu = np.asarray(gpu)
    if gpu.dtype == np.float16 or gpu.dtype == np.uint16:
        g = half_to_double(gpu)
    else:
        g = gpu.astype(np.float64)
    R = np.asarray(R, np.float64)
    tol = np.asarray(tol, np.float64)
    both_nan = np.isnan(g) & np.isnan(R)
    inf_r = np.isinf(R) | np.isinf(g)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - R)
        ratio = np.where(both_nan, 0.0, err / tol)
    ratio = np.where(inf_r & (g == R), 0.0, ratio)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    if ratio.size == 0:
        return True, 0.0, None
    idx = int(np.argmax(ratio))
    worst = float(ratio.reshape(-1)[idx])
    return bool(worst <= 1.0), worst, np.unravel_index(idx, ratio.shape)


# ---- whole-matrix checks for sizes where the full oracle is too slow ----

def checksum(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype="f32"):
    """Predicted sum of all outputs and a bound on its error.

    sum_ij (alpha A B + beta C)_ij = alpha * sum_k colsum(A)_k rowsum(B)_k
    + beta * sum_ij C_ij, in double ("From 306 ms to 86 ms" checks its results
    with the double-precision sum of C).  Returns (expected, magnitude) where
    magnitude = |alpha| sum_k colsum|A|_k rowsum|B|_k + |beta| sum|C| bounds the
    sum of the terms of G that enter the bound.
    """
    tin, tc = OPERANDS[dtype]
    A2 = _view2(A, M, K, lda, tin) if (alpha != 0 and K > 0) else None
    B2 = _view2(B, K, N, ldb, tin) if (alpha != 0 and K > 0) else None
    C2 = _view2(C, M, N, ldc, tc) if beta != 0 else None
    exp = 0.0
    mag = 0.0
    if A2 is not None:
        ca = A2.sum(axis=0)
        rb = B2.sum(axis=1)
        exp += float(alpha) * float(ca @ rb)
        mag += abs(float(alpha)) * float(np.abs(A2).sum(axis=0) @ np.abs(B2).sum(axis=1))
    if C2 is not None:
        exp += float(beta) * float(C2.sum())
        mag += abs(float(beta)) * float(np.abs(C2).sum())
    return exp, mag


def freivalds(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, x, dtype="f32"):
    """Expected y = (alpha*A*B + beta*C) @ x in double for a vector x (length
    N), formed as alpha*A(Bx) + beta*(Cx), and the magnitude vector
    |alpha| |A|(|B||x|) + |beta| |C||x| that bounds sum_j G_ij |x_j|
    (Freivalds' randomized product check)."""
    x = np.asarray(x, np.float64)
    y = np.zeros(M, np.float64)
    mag = np.zeros(M, np.float64)
    tin, tc = OPERANDS[dtype]
    if alpha != 0 and K > 0:
        A2 = _view2(A, M, K, lda, tin)
        B2 = _view2(B, K, N, ldb, tin)
        y += float(alpha) * (A2 @ (B2 @ x))
        mag += abs(float(alpha)) * (np.abs(A2) @ (np.abs(B2) @ np.abs(x)))
    if beta != 0:
        C2 = _view2(C, M, N, ldc, tc)
        y += float(beta) * (C2 @ x)
        mag += abs(float(beta)) * (np.abs(C2) @ np.abs(x))
    return y, mag


def _view2(buf, rows, cols, ld, dtype):
    """rows x cols float64 copy of a padded host buffer."""
    a = np.asarray(buf).reshape(-1)
    if dtype == "f16":
        if a.dtype == np.uint16:
            a = a.view(np.float16)
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), np.float64)
    v = np.lib.stride_tricks.as_strided(a, shape=(rows, cols), strides=(ld * a.itemsize, a.itemsize))
    if dtype == "f16":
        return half_to_double(v.view(np.uint16).copy())
    return v.astype(np.float64)
