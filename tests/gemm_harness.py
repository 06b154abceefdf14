"""Shared helpers of the GPU parity tests: upload host buffers, call the
library through its C ABI (ctypes binding), read back, compare with the
oracle element by element."""
import sys

import numpy as np

import oracle
import workloads as wl

GUARD = 512          # elements after C that must survive every call


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _np_t(dtype):
    """numpy storage type of C and of the result ("f16f32": fp32 C)."""
    return np.float16 if dtype == "f16" else np.float32


def np_in(dtype):
    """numpy storage type of A and B."""
    return np.float32 if dtype == "f32" else np.float16


def np_out(dtype):
    return _np_t(dtype)


def run(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tag="", entry=None):
    """Call gemm_f32 / gemm_f16 / gemm_f16f32 on device copies of the host buffers.

    Returns (status, C buffer after the call as a host array).  C's buffer
    is followed by a guard region of sentinels that must be left intact."""
    import torch
    import dense_gemm_fp32_amd as dg
    note("%s %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d alpha=%r beta=%r" %
         (tag, dtype, M, N, K, lda, ldb, ldc, alpha, beta))
    t = _np_t(dtype)
    dev = torch.device("cuda:0")

    def up(x):
        if x is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    dA, dB = up(A), up(B)
    cbuf = np.concatenate([np.asarray(C, t).reshape(-1), np.full(GUARD, wl.C_PAD_SENTINEL, t)])
    dC = up(cbuf)
    fn = {"f32": dg.gemm_f32, "f16": dg.gemm_f16, "f16f32": dg.gemm_f16f32}[dtype]
    if entry is not None:
        fn = getattr(dg, entry)
    stream = torch.cuda.current_stream(dev)
    rc = fn(M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, stream)
    torch.cuda.synchronize(dev)
    out = dC.cpu().numpy()
    guard = out[-GUARD:]
    assert np.array_equal(guard.view(np.uint16 if dtype == "f16" else np.uint32),
                          np.full(GUARD, wl.C_PAD_SENTINEL, t).view(np.uint16 if dtype == "f16" else np.uint32)), \
        "write past the end of C"
    return rc, out[:-GUARD]


def colmajor_buf(mat, ld, fill):
    """Column-major buffer of a rows x cols matrix: element (i, j) at
    buf[i + j*ld], pad rows i >= rows of every column filled with `fill`."""
    rows, cols = mat.shape
    buf = np.full((cols, ld), fill, dtype=mat.dtype)
    buf[:, :rows] = mat.T
    return buf.reshape(-1)


def colmajor_view(buf, rows, cols, ld):
    """rows x cols logical matrix of a column-major buffer (a copy)."""
    return np.asarray(buf).reshape(-1)[:cols * ld].reshape(cols, ld)[:, :rows].T.copy()


def run_colmajor(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tag=""):
    """Call a column-major entry point on device copies; returns (status, C
    buffer after the call).  C's buffer is followed by guard sentinels."""
    import torch
    import dense_gemm_fp32_amd as dg
    note("%s colmajor %s M=%d N=%d K=%d lda=%d ldb=%d ldc=%d" % (tag, dtype, M, N, K, lda, ldb, ldc))
    t = _np_t(dtype)
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    cbuf = np.concatenate([np.asarray(C, t).reshape(-1), np.full(GUARD, wl.C_PAD_SENTINEL, t)])
    dA, dB, dC = up(A), up(B), up(cbuf)
    fn = {"f32": dg.gemm_f32_colmajor, "f16": dg.gemm_f16_colmajor,
          "f16f32": dg.gemm_f16f32_colmajor}[dtype]
    rc = fn(M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    out = dC.cpu().numpy()
    u = np.uint16 if dtype == "f16" else np.uint32
    assert np.array_equal(out[-GUARD:].view(u), np.full(GUARD, wl.C_PAD_SENTINEL, t).view(u)), \
        "write past the end of C"
    return rc, out[:-GUARD]


def check(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out, label=""):
    """Elementwise parity of `out` (the C buffer after the call) with the
    oracle, plus: pad columns of C unchanged bit for bit.  Returns the worst
    |err|/tol."""
    R, G = oracle.gemm(M, N, K, alpha, A, lda, B, ldb, beta, C if beta != 0 else None, ldc, dtype)
    Cv = wl.view(np.asarray(C), M, N, ldc).astype(np.float64) if (beta != 0 and M and N) else 0.0
    tol = oracle.tolerance(G, np.abs(Cv), alpha, beta, K, R, oracle.out_type(dtype))
    gpu = wl.view(out, M, N, ldc)
    ok, worst, idx = oracle.compare(gpu, R, tol)
    if not ok:
        i, j = idx
        g = gpu[i, j]
        raise AssertionError("%s: worst |err|/tol = %.3g at (%d, %d): gpu %r oracle %r tol %.3g" %
                             (label, worst, i, j, g, R[i, j], tol[i, j]))
    assert_pads_unchanged(out, C, M, N, ldc, dtype)
    return worst


def assert_pads_unchanged(out, C, M, N, ldc, dtype):
    if ldc == N or M == 0:
        return
    u = np.uint16 if dtype == "f16" else np.uint32
    o = np.asarray(out).view(u).reshape(-1)
    c = np.asarray(C).view(u).reshape(-1)
    full = (M * ldc)
    o2 = o[:full].reshape(M, ldc)[:, N:]
    c2 = c[:full].reshape(M, ldc)[:, N:]
    assert np.array_equal(o2, c2), "pad columns of C were modified"


def exact_expected(dtype, R):
    """The correctly rounded result, for cases where every partial sum is exact."""
    if dtype != "f16":
        return oracle.round_f32(R)
    return oracle.round_f16(R).view(np.float16)


def bits(x, dtype):
    return np.asarray(x).view(np.uint16 if dtype == "f16" else np.uint32)


def check_sampled(dtype, w, A, B, C, out, nrows=48, seed=0, extra_rows=()):
    """Full-size parity on sampled rows (oracle on those rows only; seeded
    random rows plus `extra_rows`), the whole-matrix checksum and Freivalds'
    product check."""
    M, N, K = w.M, w.N, w.K
    rows = np.union1d(wl.sample_rows(M, nrows, seed),
                      np.array([r for r in extra_rows if 0 <= r < M], np.int64))
    t = _np_t(dtype)
    Av = wl.view(np.asarray(A), M, K, w.lda)[rows]
    Cv_full = wl.view(np.asarray(C), M, N, w.ldc)
    Csub = np.ascontiguousarray(Cv_full[rows])
    Asub = np.ascontiguousarray(Av)
    R, G = oracle.gemm(len(rows), N, K, w.alpha, Asub.reshape(-1), K, B, w.ldb, w.beta,
                       Csub.reshape(-1) if w.beta != 0 else None, N, dtype)
    tol = oracle.tolerance(G, np.abs(Csub.astype(np.float64)) if w.beta != 0 else 0.0,
                           w.alpha, w.beta, K, R, oracle.out_type(dtype))
    gpu_full = wl.view(out, M, N, w.ldc)
    ok, worst, idx = oracle.compare(np.ascontiguousarray(gpu_full[rows]), R, tol)
    assert ok, "%s sampled rows: worst %.3g at %s" % (w.name, worst, idx)
    # whole-matrix checks
    g64 = oracle.half_to_double(np.ascontiguousarray(gpu_full)) if dtype == "f16" else gpu_full.astype(np.float64)
    assert np.all(np.isfinite(g64))
    u_out = oracle.U16 if dtype == "f16" else oracle.U32
    eta = oracle.ETA16 if dtype == "f16" else oracle.ETA32
    exp, mag = oracle.checksum(M, N, K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, dtype)
    s = g64.sum()
    bound = (1 + u_out) * 4 * K * oracle.U32 * mag + u_out * np.abs(g64).sum() + M * N * eta
    assert abs(s - exp) <= bound, "checksum %r vs %r (bound %r)" % (s, exp, bound)
    x = np.random.default_rng(seed + 1).choice([-1.0, 1.0], size=N)
    y, ymag = oracle.freivalds(M, N, K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, x, dtype)
    yg = g64 @ x
    fb = (1 + u_out) * 4 * K * oracle.U32 * ymag + u_out * np.abs(g64).sum(axis=1) + N * eta
    assert np.all(np.abs(yg - y) <= fb), "Freivalds check failed"
    return worst


def layout_case(dtype, M, N, K, ta, tb, lda, ldb, ldc, seed, dist="uniform"):
    """Stored operands of a transposed-layout call and the logical matrices.

    A is stored K x M (lda >= M) when ta, else M x K; B is stored N x K
    (ldb >= K) when tb, else K x N.  Pad elements of A and B are NaN (never
    read), C's pad columns hold the sentinel.  Returns (Abuf, Bbuf, Cbuf,
    A, B, C) with A (M x K), B (K x N), C (M x N) the logical matrices."""
    t = "f32" if dtype == "f32" else "f16"
    tc = "f16" if dtype == "f16" else "f32"
    sa, sb, sc = seed, seed + 1, seed + 2
    As = wl.draw(K, M, dist, sa, t) if ta else wl.draw(M, K, dist, sa, t)
    Bs = wl.draw(N, K, dist, sb, t) if tb else wl.draw(K, N, dist, sb, t)
    C = wl.draw(M, N, dist, sc, tc)
    Abuf = wl.pad(As, lda, np.nan)
    Bbuf = wl.pad(Bs, ldb, np.nan)
    Cbuf = wl.pad(C, ldc, wl.C_PAD_SENTINEL)
    A = np.ascontiguousarray(As.T if ta else As)
    B = np.ascontiguousarray(Bs.T if tb else Bs)
    return Abuf, Bbuf, Cbuf, A, B, C


def run_layout(dtype, layout, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tag=""):
    """Call gemm_<dtype>_<layout> (layout "nt", "tn" or "tt") on device
    copies; returns (status, C buffer after the call).  C's buffer is followed
    by guard sentinels that must be left intact."""
    return run(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tag=tag + " " + layout,
               entry="gemm_%s_%s" % (dtype, layout))


def check_layout(dtype, M, N, K, alpha, A, B, beta, C, Cbuf, ldc, out, label=""):
    """Parity of a transposed-layout call's output with the oracle on the
    logical matrices (row-major copies, lda = K, ldb = N); pad columns of C
    unchanged.  Returns the worst |err|/tol."""
    R, G = oracle.gemm(M, N, K, alpha, A.reshape(-1), max(K, 1), B.reshape(-1), max(N, 1), beta,
                       np.ascontiguousarray(C).reshape(-1) if beta != 0 else None, max(N, 1), dtype)
    Cv = C.astype(np.float64) if beta != 0 else 0.0
    tol = oracle.tolerance(G, np.abs(Cv), alpha, beta, K, R, oracle.out_type(dtype))
    gpu = wl.view(out, M, N, ldc)
    ok, worst, idx = oracle.compare(gpu, R, tol)
    if not ok:
        i, j = idx
        raise AssertionError("%s: worst |err|/tol = %.3g at (%d, %d): gpu %r oracle %r tol %.3g" %
                             (label, worst, i, j, gpu[i, j], R[i, j], tol[i, j]))
    assert_pads_unchanged(out, Cbuf, M, N, ldc, dtype)
    return worst
