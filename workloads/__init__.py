"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random matrices and lays them out in padded,
row-major host buffers; it performs none of the GEMM's arithmetic.  Both the
GPU tests / benchmark and the CPU oracle take their inputs from here, so the
two sides see identical bits.

Workloads follow the shapes the pages time: square N x N fp32 products from
seeded random matrices with C zeroed before each run ("From 306 ms to 86 ms",
section on how each kernel was timed), the square fp32 size sweep
1024..12800 in steps of 128 ("Advanced Matrix Multiplication on NVIDIA GPUs"
summary, benchmarking section), an fp16-in / fp16-out GEMM standing in for
the LeetGPU problem whose shape the "LeetGPU GEMM T4" page does not give, and
fp16 inputs with an fp32 C (the tensor-core WMMA page's output type).
A ragged case with padded, unaligned leading dimensions exercises the scalar
load path and all three tails (the same summary's layout section: leading
dimensions may exceed the column count, and 128-bit loads need ld % 4 == 0).

Values: U[-1, 1] or N(0, 1) drawn in float64 by numpy's default generator
(PCG64) and rounded once to the storage type.  Pads of A and B hold NaN (a read
that leaks into the product shows up as NaN); pads of C hold a sentinel that
must survive the call unchanged.
"""
from dataclasses import dataclass, field
import math

import numpy as np

C_PAD_SENTINEL = 1234.0   # exactly representable in fp16 and fp32


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "f32" or "f16" (inputs and output), "f16f32" (fp16 in, fp32 C)
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    alpha: float
    beta: float
    dist_ab: str            # "uniform" (U[-1,1]) or "normal" (N(0,1))
    dist_c: str             # "uniform", "normal" or "zero"
    seeds: tuple            # (seed A, seed B, seed C)
    note: str = field(default="", compare=False)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K


def square(n, dtype="f32", alpha=1.0, beta=0.0, dist_c="zero", seeds=(2, 3, 4), name=None):
    return Workload(name or ("%s_%d" % (dtype, n)), dtype, n, n, n, n, n, n, alpha, beta,
                    "uniform", dist_c, tuple(seeds))


# The five workload families.
F32_256 = Workload("f32_256", "f32", 256, 256, 256, 256, 256, 256, 1.0, 0.0,
                   "uniform", "zero", (1, 2, 3), "fp32 256^3, C zeroed")
F32_SQUARE = [square(n, seeds=(2, 3, 4)) for n in (256, 512, 1024, 2048, 4096)]
F32_4096 = F32_SQUARE[-1]
F16_4096 = Workload("f16_4096_beta0.5", "f16", 4096, 4096, 4096, 4096, 4096, 4096, 1.0, 0.5,
                    "uniform", "uniform", (3, 4, 5), "fp16 in/out, fp32 accumulation")
RAGGED_F32 = Workload("ragged_f32", "f32", 1000, 3000, 517, 530, 3005, 3003, 1.5, -0.75,
                      "normal", "normal", (4, 5, 6), "lda=K+13, ldb=N+5, ldc=N+3")
RAGGED_F16 = Workload("ragged_f16", "f16", 1000, 3000, 517, 530, 3005, 3003, 1.5, -0.75,
                      "normal", "normal", (4, 5, 6), "lda=K+13, ldb=N+5, ldc=N+3")
# fp16 inputs with an fp32 C and result (the tensor-core WMMA page writes float
# accumulators from half inputs): the ragged case and the 4096^3 square.
RAGGED_F16F32 = Workload("ragged_f16f32", "f16f32", 1000, 3000, 517, 530, 3005, 3003, 1.5, -0.75,
                         "normal", "normal", (4, 5, 6), "fp16 A, B; fp32 C; lda=K+13, ldb=N+5, ldc=N+3")
F16F32_4096 = Workload("f16f32_4096_beta0.5", "f16f32", 4096, 4096, 4096, 4096, 4096, 4096, 1.0, 0.5,
                       "uniform", "uniform", (3, 4, 5), "fp16 A, B; fp32 C and result")


def sweep_sizes():
    """Square sizes 1024, 1152, ..., 12800."""
    return list(range(1024, 12800 + 1, 128))


def sweep(n):
    return square(n, alpha=1.0, beta=1.0, dist_c="uniform", seeds=(5, 6, 7),
                  name="f32_sweep_%d" % n)


ALL = [F32_256] + F32_SQUARE + [F16_4096, RAGGED_F32, RAGGED_F16, RAGGED_F16F32, F16F32_4096]


def operand_types(dtype):
    """Storage types (A and B, C) of a workload type."""
    return {"f32": ("f32", "f32"), "f16": ("f16", "f16"), "f16f32": ("f16", "f32")}[dtype]


def _np_dtype(dtype):
    return {"f32": np.float32, "f16": np.float16}[dtype]


def draw(rows, cols, dist, seed, dtype):
    """rows x cols matrix from a seeded generator, rounded once to dtype."""
    t = _np_dtype(dtype)
    if dist == "zero":
        return np.zeros((rows, cols), t)
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=(rows, cols))
    elif dist == "normal":
        x = rng.standard_normal(size=(rows, cols))
    else:
        raise ValueError(dist)
    return x.astype(t)


def pad(mat, ld, fill):
    """Place a rows x cols matrix in a rows*ld buffer (row-major, leading
    dimension ld) whose pad columns hold `fill`.  Returns the 1-D buffer."""
    rows, cols = mat.shape
    if ld < cols:
        raise ValueError("ld %d < cols %d" % (ld, cols))
    buf = np.full((rows, ld), fill, dtype=mat.dtype)
    buf[:, :cols] = mat
    return buf.reshape(-1)


def make(w, pad_ab=float("nan"), pad_c=C_PAD_SENTINEL):
    """Host buffers (A, B, C) for workload w, each 1-D and padded to its ld."""
    sa, sb, sc = w.seeds
    tin, tc = operand_types(w.dtype)
    A = pad(draw(w.M, w.K, w.dist_ab, sa, tin), w.lda, pad_ab)
    B = pad(draw(w.K, w.N, w.dist_ab, sb, tin), w.ldb, pad_ab)
    C = pad(draw(w.M, w.N, w.dist_c, sc, tc), w.ldc, pad_c)
    return A, B, C


def view(buf, rows, cols, ld):
    """rows x cols strided view of a padded 1-D buffer."""
    if rows == 0 or cols == 0:
        return buf[:0].reshape(rows, cols) if buf.size == 0 else np.zeros((rows, cols), buf.dtype)
    return np.lib.stride_tricks.as_strided(buf, shape=(rows, cols),
                                           strides=(ld * buf.itemsize, buf.itemsize))


def small_ints(rows, cols, lo, hi, seed, dtype):
    """Integer-valued matrix with entries in [lo, hi] (exactness tests)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(_np_dtype(dtype))


def odd_ints(rows, cols, hi, seed, dtype="f32"):
    """Odd integers in [-hi, hi] (12 significant bits for hi = 4095)."""
    rng = np.random.default_rng(seed)
    v = rng.integers(0, (hi + 1) // 2, size=(rows, cols)) * 2 + 1
    s = rng.choice(np.array([-1, 1]), size=(rows, cols))
    return (v * s).astype(_np_dtype(dtype))


def sample_positions(M, N, count, seed):
    """`count` distinct-ish (row, col) positions, always including the four
    corners and the last row/column, for sampled checks at full size."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, size=count))
    cols = list(rng.integers(0, N, size=count))
    rows += [0, 0, M - 1, M - 1]
    cols += [0, N - 1, 0, N - 1]
    return np.array(rows, np.int64), np.array(cols, np.int64)


def sample_rows(M, count, seed):
    """Sorted distinct row indices, including the first and last row."""
    rng = np.random.default_rng(seed)
    r = set(int(x) for x in rng.choice(M, size=min(count, M), replace=False))
    r.update({0, M - 1})
    return np.array(sorted(r), np.int64)


assert math.isclose(F32_4096.flops, 1.374389534720e11)
