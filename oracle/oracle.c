/*
 * oracle.c -- plain CPU reference for the row-major GEMM
 *
 *     C := alpha * A * B + beta * C,   A is M x K, B is K x N, C is M x N,
 *
 * evaluated in IEEE double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the GPU library.
 *
 * Sources (the web pages on hand-written GEMM kernels):
 *   - "Advanced Matrix Multiplication on NVIDIA GPUs" summary (mo.ai.kr),
 *     opening paragraphs: SGEMM computes C := alpha*A*B + beta*C.
 *     Section "memory layout and PTX": matrices are row-major, element
 *     (row, col) of an R x S matrix lives at ptr[row*S + col]; A, B and C are
 *     M x K, K x N and M x N; lda/ldb/ldc are leading dimensions, normally
 *     lda = k and ldb = ldc = n, larger when a sub-matrix is computed.
 *     Section "SGEMM tiling": the beta branch reads C only when beta != 0.
 *   - "LeetGPU GEMM T4" (currybab), baseline kernel: one output is the fp32
 *     dot product of a row of A and a column of B, then alpha*sum + beta*C,
 *     rounded once to half with the round-to-nearest conversion.
 *   - "From 306 ms to 86 ms" (kpapadogiannis), intro: each element of C is a
 *     sum of K products; section "how each kernel was timed": results are
 *     checked with the sum of all elements of C in double precision.
 *
 * Readings taken where the pages are silent (each one is listed with the
 * design notes):
 *   - alpha == 0 (or K == 0): A and B are not read; the result is beta*C.
 *   - beta == 0: C is not read (write-only), so NaN in C does not propagate.
 *   - every product is formed and summed in double, k ascending, for each
 *     output element; fp32 and fp16 inputs convert to double exactly and
 *     every fp32 x fp32 or fp16 x fp16 product is exact in double.
 *
 * Outputs: R[i*N + j] = the double result, and G[i*N + j] = sum_k |A_ik||B_kj|
 * (the magnitude term of the error bound).  Both are dense M x N arrays.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE-754 binary16 (p = 11 significand bits, emin = -14, emax = 15) ---- */

/* Decode a binary16 bit pattern into the double with the same value. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)            /* zero or subnormal: f * 2^-24 */
        v = ldexp((double)f, -24);
    else if (e == 31)      /* infinity or NaN */
        v = f ? NAN : INFINITY;
    else                   /* normal: (1 + f/1024) * 2^(e-15) */
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round a double to binary16 with round-to-nearest, ties-to-even; results
 * whose rounded magnitude exceeds the largest finite half (65504) become
 * infinity.  NaN maps to the quiet NaN 0x7e00 with the input's sign. */
uint16_t oracle_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7e00;
    double a = fabs(x);
    if (isinf(a) || a >= 131072.0)      /* far beyond the range: infinity */
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;

    /* Binade of a: a = m * 2^ue with 1 <= m < 2; subnormal halves share the
     * quantum of the lowest normal binade, 2^-24. */
    int e2;
    frexp(a, &e2);
    int ue = e2 - 1;
    if (ue < -14)
        ue = -14;
    double q = ldexp(1.0, ue - 10);     /* spacing of halves in this binade */
    double n = a / q;                   /* exact: q is a power of two */
    double fl = floor(n);
    double rem = n - fl;                /* exact */
    double nr = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        nr = fl + 1.0;
    double v = nr * q;                  /* exact, representable in binary16 range or 65536 */
    if (v > 65504.0)
        return sign | 0x7c00;
    if (v == 0.0)
        return sign;

    int e3;
    frexp(v, &e3);
    int uv = e3 - 1;
    if (uv < -14)                       /* subnormal: exponent field 0 */
        return sign | (uint16_t)ldexp(v, 24);
    uint16_t mant = (uint16_t)(ldexp(v, 10 - uv) - 1024.0);
    return sign | (uint16_t)((uv + 15) << 10) | mant;
}

/* Round a double to binary32: C's conversion is round-to-nearest-even under
 * the default floating-point environment. */
float oracle_double_to_float(double x)
{
    return (float)x;
}

/* ---- the definition, element by element ---- */

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One output row: s[j] = sum_k A(i,k) B(k,j), g[j] = sum_k |A(i,k)| |B(k,j)|,
 * k ascending.  The loop runs over k outside and j inside, which keeps the
 * per-element order of the sum (k ascending) and reads B row by row. */
static void row_f32(int N, int K, const float *Arow, const float *B, long ldb,
                    double *s, double *g)
{
    for (int j = 0; j < N; ++j) { s[j] = 0.0; g[j] = 0.0; }
    for (int k = 0; k < K; ++k) {
        double a = (double)Arow[k];
        double aa = fabs(a);
        const float *Bk = B + (size_t)k * (size_t)ldb;
        for (int j = 0; j < N; ++j) {
            double b = (double)Bk[j];
            s[j] += a * b;
            g[j] += aa * fabs(b);
        }
    }
}

/* The same row for operands already decoded to double: A's row (K values)
 * and B dense K x N.  Decoding is exact, so the sums equal those of the
 * binary16 values themselves. */
static void row_f64(int N, int K, const double *Arow, const double *B,
                    double *s, double *g)
{
    for (int j = 0; j < N; ++j) { s[j] = 0.0; g[j] = 0.0; }
    for (int k = 0; k < K; ++k) {
        double a = Arow[k];
        double aa = fabs(a);
        const double *Bk = B + (size_t)k * (size_t)N;
        for (int j = 0; j < N; ++j) {
            s[j] += a * Bk[j];
            g[j] += aa * fabs(Bk[j]);
        }
    }
}

/* A rows x cols binary16 matrix (leading dimension ld) decoded once into a
 * dense double array, so that each value is converted once per call rather
 * than once per output row.  NULL on allocation failure. */
static double *decode_dense(int rows, int cols, const uint16_t *X, long ld)
{
    double *d = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) *
                                 (size_t)(cols > 0 ? cols : 1));
    if (!d)
        return NULL;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            d[(size_t)r * (size_t)cols + c] = oracle_half_to_double(X[(size_t)r * (size_t)ld + c]);
    return d;
}

/* One output row of a binary16 product: A's row decoded into adec, then the
 * double row above against the decoded B. */
static void row_f16(int N, int K, const uint16_t *Arow, const double *Bdec,
                    double *s, double *g, double *adec)
{
    for (int k = 0; k < K; ++k)
        adec[k] = oracle_half_to_double(Arow[k]);
    row_f64(N, K, adec, Bdec, s, g);
}

/* R := alpha*A*B + beta*C and G := |A||B| for fp32 inputs.
 * A (M x K, leading dimension lda), B (K x N, ldb), C (M x N, ldc) are host
 * arrays; R and G are dense M x N.  C may be NULL when beta == 0; A and B may
 * be NULL when alpha == 0 or K == 0.  Returns 0, or -1 on allocation failure. */
int oracle_gemm_f32(int M, int N, int K, double alpha,
                    const float *A, long lda, const float *B, long ldb,
                    double beta, const float *C, long ldc,
                    double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * 2);
        if (!s) {
#pragma omp atomic write
            err = -1;
        } else {
            double *g = s + (N > 0 ? N : 1);
#pragma omp for schedule(static)
            for (int i = 0; i < M; ++i) {
                if (use_ab) {
                    row_f32(N, K, A + (size_t)i * (size_t)lda, B, ldb, s, g);
                } else {
                    for (int j = 0; j < N; ++j) { s[j] = 0.0; g[j] = 0.0; }
                }
                for (int j = 0; j < N; ++j) {
                    double r = use_ab ? alpha * s[j] : 0.0;
                    if (beta != 0.0)
                        r += beta * (double)C[(size_t)i * (size_t)ldc + j];
                    R[(size_t)i * N + j] = r;
                    G[(size_t)i * N + j] = g[j];
                }
            }
            free(s);
        }
    }
    return err;
}

/* As oracle_gemm_f32 for binary16 inputs and C (bit patterns). */
int oracle_gemm_f16(int M, int N, int K, double alpha,
                    const uint16_t *A, long lda, const uint16_t *B, long ldb,
                    double beta, const uint16_t *C, long ldc,
                    double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
    int err = 0;
    double *bdec = NULL;
    if (use_ab && M > 0) {
        bdec = decode_dense(K, N, B, ldb);
        if (!bdec)
            return -1;
    }
#pragma omp parallel
    {
        size_t n1 = (size_t)(N > 0 ? N : 1);
        size_t k1 = (size_t)(K > 0 ? K : 1);
        double *s = (double *)malloc(sizeof(double) * (n1 * 2 + k1));
        if (!s) {
#pragma omp atomic write
            err = -1;
        } else {
            double *g = s + n1;
            double *adec = s + 2 * n1;
#pragma omp for schedule(static)
            for (int i = 0; i < M; ++i) {
                if (use_ab) {
                    row_f16(N, K, A + (size_t)i * (size_t)lda, bdec, s, g, adec);
                } else {
                    for (int j = 0; j < N; ++j) { s[j] = 0.0; g[j] = 0.0; }
                }
                for (int j = 0; j < N; ++j) {
                    double r = use_ab ? alpha * s[j] : 0.0;
                    if (beta != 0.0)
                        r += beta * oracle_half_to_double(C[(size_t)i * (size_t)ldc + j]);
                    R[(size_t)i * N + j] = r;
                    G[(size_t)i * N + j] = g[j];
                }
            }
            free(s);
        }
    }
    free(bdec);
    return err;
}

/* Mixed precision: binary16 A and B, binary32 C (and output).  The page on
 * tensor-core WMMA versus fp32 cores accumulates half products into float
 * accumulators and writes the float result; here, as everywhere in this
 * file, the sum is formed in double (every half product is exact), and C is
 * read as float only when beta != 0. */
int oracle_gemm_f16f32(int M, int N, int K, double alpha,
                       const uint16_t *A, long lda, const uint16_t *B, long ldb,
                       double beta, const float *C, long ldc,
                       double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
    int err = 0;
    double *bdec = NULL;
    if (use_ab && M > 0) {
        bdec = decode_dense(K, N, B, ldb);
        if (!bdec)
            return -1;
    }
#pragma omp parallel
    {
        size_t n1 = (size_t)(N > 0 ? N : 1);
        size_t k1 = (size_t)(K > 0 ? K : 1);
        double *s = (double *)malloc(sizeof(double) * (n1 * 2 + k1));
        if (!s) {
#pragma omp atomic write
            err = -1;
        } else {
            double *g = s + n1;
            double *adec = s + 2 * n1;
#pragma omp for schedule(static)
            for (int i = 0; i < M; ++i) {
                if (use_ab) {
                    row_f16(N, K, A + (size_t)i * (size_t)lda, bdec, s, g, adec);
                } else {
                    for (int j = 0; j < N; ++j) { s[j] = 0.0; g[j] = 0.0; }
                }
                for (int j = 0; j < N; ++j) {
                    double r = use_ab ? alpha * s[j] : 0.0;
                    if (beta != 0.0)
                        r += beta * (double)C[(size_t)i * (size_t)ldc + j];
                    R[(size_t)i * N + j] = r;
                    G[(size_t)i * N + j] = g[j];
                }
            }
            free(s);
        }
    }
    free(bdec);
    return err;
}

/* Selected elements only: R[t], G[t] for (rows[t], cols[t]), t < count.  Same
 * arithmetic as the full version (k ascending), for sizes where the full
 * product would take too long on the host. */
void oracle_gemm_f32_elems(int K, double alpha,
                           const float *A, long lda, const float *B, long ldb,
                           double beta, const float *C, long ldc,
                           long count, const long *rows, const long *cols,
                           double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
#pragma omp parallel for schedule(static)
    for (long t = 0; t < count; ++t) {
        size_t i = (size_t)rows[t], j = (size_t)cols[t];
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int k = 0; k < K; ++k) {
                double a = (double)A[i * (size_t)lda + k];
                double b = (double)B[(size_t)k * (size_t)ldb + j];
                s += a * b;
                g += fabs(a) * fabs(b);
            }
        }
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0)
            r += beta * (double)C[i * (size_t)ldc + j];
        R[t] = r;
        G[t] = g;
    }
}

void oracle_gemm_f16_elems(int K, double alpha,
                           const uint16_t *A, long lda, const uint16_t *B, long ldb,
                           double beta, const uint16_t *C, long ldc,
                           long count, const long *rows, const long *cols,
                           double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
#pragma omp parallel for schedule(static)
    for (long t = 0; t < count; ++t) {
        size_t i = (size_t)rows[t], j = (size_t)cols[t];
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int k = 0; k < K; ++k) {
                double a = oracle_half_to_double(A[i * (size_t)lda + k]);
                double b = oracle_half_to_double(B[(size_t)k * (size_t)ldb + j]);
                s += a * b;
                g += fabs(a) * fabs(b);
            }
        }
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0)
            r += beta * oracle_half_to_double(C[i * (size_t)ldc + j]);
        R[t] = r;
        G[t] = g;
    }
}

void oracle_gemm_f16f32_elems(int K, double alpha,
                              const uint16_t *A, long lda, const uint16_t *B, long ldb,
                              double beta, const float *C, long ldc,
                              long count, const long *rows, const long *cols,
                              double *R, double *G)
{
    int use_ab = (alpha != 0.0) && (K > 0);
#pragma omp parallel for schedule(static)
    for (long t = 0; t < count; ++t) {
        size_t i = (size_t)rows[t], j = (size_t)cols[t];
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int k = 0; k < K; ++k) {
                double a = oracle_half_to_double(A[i * (size_t)lda + k]);
                double b = oracle_half_to_double(B[(size_t)k * (size_t)ldb + j]);
                s += a * b;
                g += fabs(a) * fabs(b);
            }
        }
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0)
            r += beta * (double)C[i * (size_t)ldc + j];
        R[t] = r;
        G[t] = g;
    }
}

/* Bulk conversions used by the Python side. */
void oracle_round_to_half(long count, const double *x, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (long t = 0; t < count; ++t)
        out[t] = oracle_double_to_half(x[t]);
}

void oracle_half_to_double_array(long count, const uint16_t *h, double *out)
{
#pragma omp parallel for schedule(static)
    for (long t = 0; t < count; ++t)
        out[t] = oracle_half_to_double(h[t]);
}
