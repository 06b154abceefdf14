"""ctypes binding of libgemm.so: the C entry points of include/gemm.h under
the same names, plus a torch-tensor convenience wrapper.

Only argument marshalling happens here; every step of the GEMM runs in the
HIP kernels of libgemm.so.  There is no fallback: if the library is missing
the import fails with an error that says how to build it.
"""
import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first, so libgemm.so binds to the same one)

HERE = os.path.dirname(os.path.abspath(__file__))
# DENSE_GEMM_FP32_AMD_LIB selects another build of the same library (the
# LDS-poison debug build of build.py); by default the release build next to
# this file.
LIB_PATH = os.environ.get("DENSE_GEMM_FP32_AMD_LIB") or os.path.join(HERE, "libgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgemm.so is not built (%s); run `python -m dense_gemm_fp32_amd.build`"
                      % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_I = ctypes.c_int
_F = ctypes.c_float
_P = ctypes.c_void_p

_lib.gemm_f32.argtypes = [_I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, _P]
_lib.gemm_f32.restype = _I
_lib.gemm_f16.argtypes = [_I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, _P]
_lib.gemm_f16.restype = _I
_lib.gemm_f16f32.argtypes = [_I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, _P]
_lib.gemm_f16f32.restype = _I
LAYOUT_NAMES = tuple("gemm_%s_%s" % (t, l) for t in ("f32", "f16", "f16f32") for l in ("nt", "tn", "tt"))
for _n in ("gemm_f32_colmajor", "gemm_f16_colmajor", "gemm_f16f32_colmajor",
           "gemm_f32_valu", "gemm_f32_noalloc") + LAYOUT_NAMES:
    getattr(_lib, _n).argtypes = [_I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, _P]
    getattr(_lib, _n).restype = _I
_lib.gemm_status_string.argtypes = [_I]
_lib.gemm_status_string.restype = ctypes.c_char_p
_lib.gemm_describe.argtypes = [_I, _I, _I, _I, _F, _P, _I, _P, _I, _F, _P, _I, ctypes.c_char_p, _I]
_lib.gemm_describe.restype = _I
_lib.gemm_set_load_mode.argtypes = [_I]
_lib.gemm_set_load_mode.restype = _I
_lib.gemm_set_tile_config.argtypes = [_I]
_lib.gemm_set_tile_config.restype = _I
_lib.gemm_set_split.argtypes = [_I]
_lib.gemm_set_split.restype = _I
_lib.gemm_set_tail_split.argtypes = [_I]
_lib.gemm_set_tail_split.restype = _I
_lib.gemm_set_pack.argtypes = [_I]
_lib.gemm_set_pack.restype = _I
_lib.gemm_set_stream_k.argtypes = [_I]
_lib.gemm_set_stream_k.restype = _I
_lib.gemm_set_workspace_limit.argtypes = [ctypes.c_longlong]
_lib.gemm_set_workspace_limit.restype = ctypes.c_longlong
_lib.gemm_probe_mfma.argtypes = [_I, _I, _P, ctypes.c_size_t, _P, ctypes.c_size_t,
                                 ctypes.POINTER(ctypes.c_double), _P]
_lib.gemm_probe_mfma.restype = _I

EXPORTS = ("gemm_f32", "gemm_f16", "gemm_f16f32", "gemm_f32_valu", "gemm_f32_noalloc",
           "gemm_f32_colmajor", "gemm_f16_colmajor", "gemm_f16f32_colmajor", "gemm_status_string",
           "gemm_describe", "gemm_set_load_mode", "gemm_set_tile_config", "gemm_set_split",
           "gemm_set_tail_split", "gemm_set_pack", "gemm_set_stream_k", "gemm_set_workspace_limit",
           "gemm_probe_mfma") + LAYOUT_NAMES
GEMM_ERR_SCRATCH_LIMIT = -200


class GemmError(RuntimeError):
    def __init__(self, status):
        super().__init__("gemm status %d: %s" % (status, gemm_status_string(status)))
        self.status = status


def _addr(x):
    """Device address of a torch tensor, or an integer address as given."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return None
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C := alpha*A*B + beta*C in fp32 (see include/gemm.h).  A, B, C are
    device addresses or torch tensors; stream is a hipStream_t handle, a
    torch.cuda.Stream or None (the null stream).  Returns the status code."""
    return _lib.gemm_f32(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                         _stream(stream))


def gemm_f16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """fp16-in / fp16-out GEMM with fp32 accumulation (see include/gemm.h)."""
    return _lib.gemm_f16(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                         _stream(stream))


def gemm_f16f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """fp16 A and B, fp32 C and result, fp32 accumulation (see include/gemm.h)."""
    return _lib.gemm_f16f32(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                            _stream(stream))


def gemm_f32_valu(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """fp32 GEMM on the vector ALUs (ablation of the matrix-core path; see
    include/gemm.h)."""
    return _lib.gemm_f32_valu(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                              _stream(stream))


def gemm_f32_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """gemm_f32 with its split-K workspace in the library's fixed scratch
    region: no allocation (see include/gemm.h); GEMM_ERR_SCRATCH_LIMIT when
    the call would need more workspace than the region holds."""
    return _lib.gemm_f32_noalloc(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C),
                                 ldc, _stream(stream))


def gemm_f32_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """Column-major (BLAS layout) fp32 GEMM (see include/gemm.h)."""
    return _lib.gemm_f32_colmajor(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C),
                                  ldc, _stream(stream))


def gemm_f16_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """Column-major fp16 GEMM with fp32 accumulation (see include/gemm.h)."""
    return _lib.gemm_f16_colmajor(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C),
                                  ldc, _stream(stream))


def gemm_f16f32_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """Column-major fp16 A and B with an fp32 C (see include/gemm.h)."""
    return _lib.gemm_f16f32_colmajor(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                     _addr(C), ldc, _stream(stream))


def gemm_status_string(status):
    return _lib.gemm_status_string(int(status)).decode()


def gemm_describe(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    """(status, text) describing the variant chosen for these arguments."""
    buf = ctypes.create_string_buffer(256)
    dt = {"f32": 0, "f16": 1, "f16f32": 2}.get(dtype, dtype)
    rc = _lib.gemm_describe(dt, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                            buf, len(buf))
    return rc, buf.value.decode()


def gemm_set_load_mode(mode):
    """0 = vector/scalar loads by alignment (default), 1 = force scalar."""
    return _lib.gemm_set_load_mode(int(mode))


def gemm_set_tile_config(config):
    """0 = tile configuration by problem size (default); 1/2/3/4 = force the
    large/medium/small/tiny configuration (fp16 maps 4 to small); 5 = fp32
    medium with loads issued together; 6 = fp32 256x256 (fp16 large on
    32x32x16 blocks); 7 = fp32 64x64 with four waves (fp16 small); 8 = fp32
    128x64 with four waves (fp16 medium); 9 = fp32 64x64 with four waves in
    64-k steps (fp16 small); 10 = fp32 32x32, one wave, 64-k steps (fp16
    small)."""
    return _lib.gemm_set_tile_config(int(config))


def _layout_entry(name):
    fn = getattr(_lib, name)

    def call(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
        return fn(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                  _stream(stream))
    call.__name__ = name
    call.__doc__ = ("%s: C := alpha*op(A)*op(B) + beta*C with the operand layouts its suffix "
                    "names (see include/gemm.h).  Returns the status code." % name)
    return call


for _n in LAYOUT_NAMES:
    globals()[_n] = _layout_entry(_n)


def gemm_probe_mfma(dtype, iters, operands, out, stream=None):
    """Matrix-core ceiling probe (see include/gemm.h): `operands` and `out`
    are device torch tensors (at least 64 KiB and 1 MiB).  Returns (status,
    flops of the launch)."""
    flops = ctypes.c_double(0.0)
    rc = _lib.gemm_probe_mfma(int(dtype), int(iters), _addr(operands),
                              operands.numel() * operands.element_size(), _addr(out),
                              out.numel() * out.element_size(), ctypes.byref(flops),
                              _stream(stream))
    return rc, flops.value


def gemm_set_tail_split(mode):
    """fp32: 0 = split the last partly filled round of tiles by size
    (default), 1 = never, 2..64 = force that many K chunks for it."""
    return _lib.gemm_set_tail_split(int(mode))


def gemm_set_pack(mode):
    """0 = copy operands whose rows do not allow 16-byte loads to 16-byte rows
    in fp32 calls of at least 5e9 flops, or 1.5e9 with N % 4 == 0 (default);
    1 = never; 2 = whenever their rows do not allow 16-byte loads (fp16
    too).  Returns the previous mode, or -1."""
    return _lib.gemm_set_pack(int(mode))


def gemm_set_stream_k(mode):
    """fp32: 0 = Stream-K by size (default), 1 = never; with the 64x64
    four-wave tile or a forced tile configuration (1, 5, 6, 7): 2..4 = every
    tile's K steps over 1..3 workgroups per CU, 5..6 = whole rounds first,
    the rest over 1..2 more workgroups per CU.  Returns the previous mode,
    or -1."""
    return _lib.gemm_set_stream_k(int(mode))


def gemm_set_workspace_limit(nbytes):
    """Cap on one call's split-K workspace from the pool: -1 = none
    (default), 0 = never split, n = splits needing more than n bytes run
    unsplit.  Returns the previous setting."""
    return _lib.gemm_set_workspace_limit(int(nbytes))


def gemm_set_split(mode):
    """0 = split K by problem size (default), 1 = never, 2..64 = force that
    many K chunks."""
    return _lib.gemm_set_split(int(mode))


def _operand(name, t):
    """(transposed, ld) of a 2-D operand: rows contiguous (stride(1) == 1) as
    stored, or columns contiguous (stride(0) == 1: the transpose of a
    row-major tensor, e.g. X.t())."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    rows, cols = t.shape
    if t.stride(1) == 1 and (t.stride(0) >= cols or rows <= 1):
        return False, max(t.stride(0), cols, 1)
    if t.stride(0) == 1 and (t.stride(1) >= rows or cols <= 1):
        return True, max(t.stride(1), rows, 1)
    raise ValueError("%s must have contiguous rows (stride(1) == 1) or contiguous columns "
                     "(stride(0) == 1)" % name)


def gemm(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C := alpha*A@B + beta*C for 2-D torch tensors on the GPU (in place).

    A and B may be row-major (stride(1) == 1, rows possibly padded) or
    transposed views of row-major tensors (stride(0) == 1, e.g. X.t()); the
    latter run the _nt / _tn / _tt entry points, which read the operand in
    its stored orientation.  C must have stride(1) == 1.  float32 tensors go
    to the fp32 entry points, float16 to the fp16 ones, float16 A and B with a
    float32 C to the fp16-in / fp32-out ones.  Uses the current torch stream
    unless one is given."""
    ta, lda = _operand("A", A)
    tb, ldb = _operand("B", B)
    if C.dim() != 2 or C.stride(1) != 1 or (C.shape[0] > 1 and C.stride(0) < C.shape[1]):
        raise ValueError("C must be 2-D with stride(1) == 1 and stride(0) >= its column count")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                             tuple(C.shape)))
    if A.dtype != B.dtype:
        raise ValueError("A and B must share a dtype")
    if A.dtype not in (torch.float32, torch.float16):
        raise ValueError("unsupported dtype %s" % A.dtype)
    mixed = A.dtype == torch.float16 and C.dtype == torch.float32
    if C.dtype != A.dtype and not mixed:
        raise ValueError("C must have A's dtype, or float32 with float16 A and B")
    if not (A.is_cuda and B.is_cuda and C.is_cuda):
        raise ValueError("A, B and C must be GPU tensors")
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    ldc = max(C.stride(0), N, 1)
    kind = "f32" if A.dtype == torch.float32 else ("f16f32" if mixed else "f16")
    name = "gemm_" + kind + ("" if not (ta or tb) else "_" + ("t" if ta else "n") + ("t" if tb else "n"))
    rc = globals()[name](M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    if rc != 0:
        raise GemmError(rc)
    return C
