"""Host-side performance model of the GEMM: algorithmic work and bytes, the
tile re-read traffic model, LDS budgets and the benchmark replay schedule.
Pure arithmetic on sizes; imports nothing from the GPU library."""
import math

# MI355X (gfx950) published peaks.
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6}
PEAK_HBM_GBS = 8000.0
LDS_BYTES_PER_CU = 160 * 1024


def flops(M, N, K):
    """2 flops (one multiply, one add) per term of every output's sum."""
    return 2.0 * M * N * K


def algorithmic_bytes(M, N, K, elem_bytes, beta_nonzero):
    """Compulsory HBM traffic: read A and B once, write C once, and read C once
    more when beta != 0."""
    return elem_bytes * (M * K + K * N) + elem_bytes * M * N * (2 if beta_nonzero else 1)


def global_reads_per_output(K, tile_m, tile_n):
    """Global-memory element reads per output element when each tile_m x tile_n
    block of C streams its A row panel (tile_m x K) and B column panel
    (K x tile_n) once: (tile_m*K + K*tile_n) / (tile_m*tile_n).  One thread per
    output (1 x 1 tiles) reads 2K ("From 306 ms to 86 ms": 8192 at N = 4096,
    512 with 16 x 16 tiles, 256 with 32 x 32)."""
    return K / tile_n + K / tile_m


def staged_bytes(M, N, K, tile_m, tile_n, elem_bytes):
    """Bytes moved from L2/HBM into LDS over the whole GEMM with tile_m x tile_n
    workgroup tiles (the re-read traffic; served mostly by the caches)."""
    return elem_bytes * M * N * global_reads_per_output(K, tile_m, tile_n)


def lds_tile_bytes(tile_m, tile_n, tile_k, elem_bytes, stages=1, pad_a=0, pad_b=0):
    """LDS bytes for `stages` copies of an A tile (tile_m x tile_k) and a B tile
    (tile_k x tile_n), with optional per-row padding in elements.  The
    "LeetGPU GEMM T4" page's coarsened kernel (128 x 128 outputs as a 256-row
    A panel and 128-column B panel, K step 32, fp32 staging) needs
    4 * 32 * 32 * (8 + 4) bytes = 48 KB."""
    a = tile_m * (tile_k + pad_a)
    b = tile_k * (tile_n + pad_b)
    return elem_bytes * (a + b) * stages


def replay_count(n):
    """Replays per size of the unlocked-clock protocol in the SGEMM summary's
    benchmarking section: floor(1000 * exp((1024 - n) / 3100)); the mean of
    the second half of the runs is reported."""
    return int(math.floor(1000.0 * math.exp((1024.0 - n) / 3100.0)))


def replays_averaged(n):
    return replay_count(n) // 2
