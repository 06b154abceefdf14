/*
 * gemm.h -- C ABI of the MI355X (gfx950) dense GEMM library, libgemm.so.
 *
 * Operation (every entry point):
 *
 *     C := alpha * A * B + beta * C
 *
 * with A an M x K matrix, B a K x N matrix and C an M x N matrix, all
 * row-major with leading dimensions: element (i, j) of X is X[i*ldX + j].
 * This is the SGEMM definition and layout of the "Advanced Matrix
 * Multiplication on NVIDIA GPUs" summary (opening paragraphs and the section
 * on memory layout: row-major storage, lda = k and ldb = ldc = n for dense
 * matrices, larger leading dimensions for sub-matrices or padded rows).
 * gemm_f16 is the fp16-in / fp16-out variant with fp32 accumulation that the
 * "LeetGPU GEMM T4" page solves: products are summed in fp32, alpha*sum +
 * beta*C is formed in fp32 and rounded once to half, round-to-nearest-even.
 * gemm_f16f32 takes fp16 A and B with an fp32 C and result: the float
 * accumulators of the "Tensorcore_wmma_vs_fp32 test code" page, whose WMMA
 * kernel multiplies half fragments into float accumulators and stores those.
 *
 * Semantics:
 *   - beta == 0: C is write-only; its previous contents (NaN included) are
 *     never read (the tiling section of the SGEMM summary reads C only when
 *     beta != 0).
 *   - alpha == 0 or K == 0: A and B are not read; C := beta * C (beta == 0
 *     writes zeros without reading C; beta == 1 returns without launching).
 *   - M == 0 or N == 0: nothing to do; returns 0 without launching.
 *   - The summation order over K is fixed for a given shape, leading
 *     dimensions and alignment, so repeated calls give bitwise-identical
 *     results: no atomics, and a call that splits K (below) sums its chunks
 *     in a fixed order.
 *   - Split K: when a problem's tile grid would leave CUs idle, a call may
 *     divide K into S chunks, multiply each chunk into its own fp32 slab of a
 *     workspace, and then form alpha * (slab_0 + ... + slab_{S-1}) + beta * C
 *     in one more pass (same bound; one rounding to the output type).  An
 *     fp32 call whose tiles fill some whole rounds of the CUs and leave a
 *     small remainder may do this for the remainder's tiles only (dense
 *     per-tile blocks of the workspace, S * tiles * BM * BN floats), after
 *     the whole rounds.
 *   - Stream-K (fp32): when the tiles a call takes leave the last round of
 *     the CUs partly filled -- 64x64 tiles past two whole rounds with at most
 *     half a round more, or past three with at most a third of a round more
 *     (K <= 2 max(M, N)); 128x64 tiles over two to three and a half rounds
 *     (M, N, K >= 640); 256x256 tiles wherever there is a round of them and
 *     97% of their area lies inside the matrix; 128x128 tiles over 2 to 7
 *     rounds (up to 16 where the size rules pick that tile anyway) with a
 *     quarter to seven eighths of a round more; the 256x128 tile whenever it
 *     is picked; for the larger tiles 1024 <= K <= 2 max(M, N) --
 *     the whole rounds' tiles run whole while the remainder's K steps are
 *     dealt out evenly, in runs that may span two tiles, to one more
 *     workgroup per CU in the same launch (the "Stream-K" decomposition that
 *     the SGEMM summary's results section names).  A tile so shared is
 *     summed from its parts' fp32 partial sums, in K order, by a second pass
 *     that also applies alpha and beta (two fp32 tile blocks of workspace per
 *     Stream-K workgroup: 8, 16, 32, 64 or 128 MiB by tile).
 *   - Operand copies (fp32): when the rows of A or B do not allow 16-byte
 *     loads (ld not a multiple of 4, or a base not 16-byte aligned) and the
 *     call does at least 5e9 flops, or 1.5e9 with N a multiple of 4, that
 *     operand is first copied, bit for bit, into workspace rows padded to 16
 *     bytes, and the GEMM runs on the copy (the SGEMM summary's
 *     memory-layout section: its 128-bit loads need ld % 4 == 0).  Same
 *     products, same bound; the tile and split are chosen for the copy.
 *     Smaller calls, fp16 calls (unless forced, gemm_set_pack) and calls
 *     whose workspace cannot be had load such operands in pairs or element
 *     by element instead.
 *   - Accuracy: |C_gpu - C_exact| <= 4*K*u*(|alpha|*(|A||B|)_ij + |beta|*|C_ij|)
 *     plus one rounding to the output type, u = 2^-24 (fp32 accumulation).
 *
 * Memory and ownership:
 *   - A, B and C are DEVICE pointers owned by the caller.  The library keeps
 *     no pointer to them after it returns and never allocates or frees the
 *     caller's memory.
 *   - A split-K call needs S*M*ceil(N/4)*16 bytes of workspace (a last-round
 *     split S*tiles*BM*BN*4 bytes, a Stream-K call 2*64*64*4 bytes per
 *     Stream-K workgroup; at most 1 GiB, larger splits are not taken) and takes it from a memory pool the library creates per device,
 *     with stream-ordered allocation on the call's stream, returning it to
 *     the pool, in stream order, after its last kernel.  Requests are made at
 *     the largest size used so far on the device up to 256 MiB (2 MiB
 *     steps), so that freed blocks are reused, and larger ones at their own
 *     size; the pool keeps up to 256 MiB of freed blocks and hands the rest
 *     back to the runtime at the next synchronisation.
 *     Operand copies (above) take rows*ceil(cols/v)*16 bytes each (v = 4
 *     floats or 8 halves per 16 bytes) from the same allocation as the
 *     split.  gemm_set_workspace_limit caps the workspace of a call.  If the
 *     workspace cannot be had the call runs without copies or splitting (same
 *     bound; the summation order is then that of an unsplit call).
 *     gemm_describe reports the workspace a call would take.
 *   - gemm_f32_noalloc is gemm_f32 without any allocation: its workspace is a
 *     fixed 64 MiB region of device memory owned by the library (one per
 *     device, held until the process ends).
 *   - C must not overlap A or B.
 *   - The pad elements of each row (columns K..lda-1 of A, N..ldb-1 of B,
 *     N..ldc-1 of C) are never read or written.
 *
 * Streams and synchronisation:
 *   - `stream` is a hipStream_t (NULL = the default stream).  The call only
 *     enqueues work on it and returns; it does not synchronise.  The caller
 *     keeps A, B and C alive until that work has completed.
 *   - Calls may be captured into a HIP graph on a capturing stream (no
 *     memset is enqueued; the workspace of a split or operand-copying call
 *     becomes the graph's allocation node); replays repeat the captured
 *     arguments and choice.
 *   - The library keeps no per-call state, so calls are thread-safe and
 *     reentrant; the only process-wide state is the workspace pools and the
 *     diagnostic switches at the end of this header (default off).
 *
 * Return value:
 *   0                 success (work enqueued, or nothing to do)
 *   -i (i = 1..12)    argument i (1-based, in signature order) is invalid.
 *                     Checks run in this order and the first failure wins
 *                     (row-major entry points; see the column-major ones
 *                     below for their leading-dimension rules):
 *                       M < 0 -> -1, N < 0 -> -2, K < 0 -> -3,
 *                       lda < max(1, K) -> -6, ldb < max(1, N) -> -8,
 *                       ldc < max(1, N) -> -11,
 *                       A == NULL -> -5, B == NULL -> -7 (only when A and B
 *                       would be read: M, N > 0, K > 0, alpha != 0),
 *                       C == NULL -> -10 (only when M, N > 0 and C would be
 *                       touched).
 *                     Argument checks make no HIP call, so they work without
 *                     a GPU.
 *   > 0               a hipError_t from the kernel launch.
 *   GEMM_ERR_SCRATCH_LIMIT (gemm_f32_noalloc only) the call would need more
 *                     split-K workspace than the fixed scratch region holds
 *                     (operand copies are made only where they fit);
 *                     nothing was enqueued.
 */
#ifndef DENSE_GEMM_GEMM_H
#define DENSE_GEMM_GEMM_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE-754 binary16 bit pattern (1 sign, 5 exponent, 10 fraction bits). */
typedef uint16_t gemm_half_t;

#define GEMM_SUCCESS 0
#define GEMM_ERR_SCRATCH_LIMIT (-200)

/*
 * fp32 GEMM: A, B, C hold binary32 values; products are accumulated in fp32
 * on the matrix cores (v_mfma_f32_32x32x2_f32), then alpha*acc + beta*C is
 * formed in fp32 and stored.
 *   M, N, K        problem size (>= 0)
 *   alpha, beta    scalars (binary32)
 *   A, lda         device pointer to A (M x K), lda >= max(1, K)
 *   B, ldb         device pointer to B (K x N), ldb >= max(1, N)
 *   C, ldc         device pointer to C (M x N), ldc >= max(1, N); in/out
 *   stream         hipStream_t to enqueue on (NULL = default stream)
 */
int gemm_f32(int M, int N, int K, float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta, float *C, int ldc,
             void *stream);

/*
 * fp16 GEMM with fp32 accumulation: A, B, C hold binary16 bit patterns;
 * products are exact in fp32 and accumulated in fp32 on the matrix cores
 * (v_mfma_f32_16x16x32_f16 on the large tile, v_mfma_f32_32x32x16_f16 on the
 * smaller ones); alpha*acc + beta*C is formed in fp32 (C widened
 * exactly) and rounded once to binary16, round-to-nearest-even, overflowing
 * to +-infinity.  Arguments as for gemm_f32; alpha and beta are binary32.
 */
int gemm_f16(int M, int N, int K, float alpha,
             const gemm_half_t *A, int lda,
             const gemm_half_t *B, int ldb,
             float beta, gemm_half_t *C, int ldc,
             void *stream);

/*
 * fp16 inputs, fp32 C and result: A and B hold binary16 values (as for
 * gemm_f16), C holds binary32.  Products are accumulated in fp32 on the
 * matrix cores (as for gemm_f16); alpha*acc + beta*C is formed in fp32
 * and stored as binary32 (no rounding to half).  Arguments and return values
 * as for gemm_f32, with ldc counting floats.  The degenerate paths (alpha == 0
 * or K == 0) scale the fp32 C as gemm_f32 does.
 */
int gemm_f16f32(int M, int N, int K, float alpha,
                const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb,
                float beta, float *C, int ldc,
                void *stream);

/*
 * gemm_f32 for callers that cannot allocate device memory: code under HIP
 * graph capture that must not add allocation nodes, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, semantics, plan, kernels
 * and results (bit for bit) as gemm_f32; the caller still passes A, B and C.
 * The only difference is where a split-K call's workspace comes from: a
 * file-scope device array of 64 MiB inside the library (one copy per device,
 * held until the process ends) instead of the memory pool, so the call makes
 * no hipMalloc, hipFree or pool allocation.  A call whose plan would need
 * more workspace than that returns GEMM_ERR_SCRATCH_LIMIT before enqueuing
 * anything (gemm_describe reports the workspace a call would take).  Nothing
 * in the region needs to start at zero: every split pass writes the values
 * its reduction reads.  All calls on one device share the region, which keeps
 * the last call's contents: calls that may overlap on one device (different
 * streams without ordering between them) race on it, so order them (one
 * stream, or events).  The first call on a device looks up the region's
 * address there (hipGetSymbolAddress).
 */
int gemm_f32_noalloc(int M, int N, int K, float alpha,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float beta, float *C, int ldc,
                     void *stream);

/*
 * fp32 GEMM on the vector ALUs instead of the matrix cores: the SIMT design of
 * the pages' SGEMM kernels (shared-memory tiles, 8 x 8 outputs per thread in
 * registers: "From 306 ms to 86 ms", register blocking, and the SGEMM
 * summary's tiling section), kept as the ablation against gemm_f32.  Same
 * arguments, semantics and return values as gemm_f32; fp32 FMAs (no packed
 * form) against the 157.3 TFLOP/s fp32 vector peak.  Never splits K and
 * takes no workspace.
 */
int gemm_f32_valu(int M, int N, int K, float alpha,
                  const float *A, int lda,
                  const float *B, int ldb,
                  float beta, float *C, int ldc,
                  void *stream);

/*
 * Column-major variants (BLAS layout): element (i, j) of X is X[i + j*ldX],
 * with lda >= max(1, M), ldb >= max(1, K), ldc >= max(1, M).  Same operation,
 * semantics, precisions, ownership, streams and return values as the
 * row-major entry points above; the argument checks use these column-major
 * rules (-6 for lda < max(1, M), -8 for ldb < max(1, K), -11 for
 * ldc < max(1, M), the rest as above).  A column-major matrix is the
 * row-major matrix of its transpose on the same bytes, so each call runs the
 * row-major product C^T = B^T * A^T: the "Advanced Matrix Multiplication on
 * NVIDIA GPUs" summary's layout section handles column-major use by swapping
 * A and B in the same way.
 */
int gemm_f32_colmajor(int M, int N, int K, float alpha,
                      const float *A, int lda,
                      const float *B, int ldb,
                      float beta, float *C, int ldc,
                      void *stream);
int gemm_f16_colmajor(int M, int N, int K, float alpha,
                      const gemm_half_t *A, int lda,
                      const gemm_half_t *B, int ldb,
                      float beta, gemm_half_t *C, int ldc,
                      void *stream);
int gemm_f16f32_colmajor(int M, int N, int K, float alpha,
                         const gemm_half_t *A, int lda,
                         const gemm_half_t *B, int ldb,
                         float beta, float *C, int ldc,
                         void *stream);

/*
 * Transposed operands, row-major storage: C := alpha * op(A) * op(B) + beta*C
 * with op(A) M x K and op(B) K x N.  The suffix gives the operations, A's
 * first: "n" = the operand as stored, "t" = its transpose.
 *   _nt: A is M x K (lda >= max(1, K)); B is stored N x K (ldb >= max(1, K)),
 *        op(B) = B^T (element (k, n) of op(B) is B[n*ldb + k]);
 *   _tn: A is stored K x M (lda >= max(1, M)), op(A) = A^T (element (m, k)
 *        of op(A) is A[k*lda + m]); B is K x N (ldb >= max(1, N));
 *   _tt: both stored transposed (lda >= max(1, M), ldb >= max(1, K)).
 * C is M x N, ldc >= max(1, N).  The SGEMM summary's layout section covers
 * row-major storage and column-major use (by swapping A and B); these are
 * BLAS's other operand forms, the transposes, on row-major storage, done
 * natively: each operand sits in LDS in its stored orientation and the
 * matrix-core fragments are read from it (no transposed copy is made).  Same
 * semantics, precisions, accuracy bound, ownership, streams and split-K
 * behaviour as the plain entry points; the argument checks use the row
 * lengths above (-6 for lda, -8 for ldb, -11 for ldc, the rest as for
 * gemm_f32).
 */
int gemm_f32_nt(int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, void *stream);
int gemm_f32_tn(int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, void *stream);
int gemm_f32_tt(int M, int N, int K, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, void *stream);
int gemm_f16_nt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc,
                void *stream);
int gemm_f16_tn(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc,
                void *stream);
int gemm_f16_tt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc,
                void *stream);
int gemm_f16f32_nt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc,
                   void *stream);
int gemm_f16f32_tn(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc,
                   void *stream);
int gemm_f16f32_tt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc,
                   void *stream);

/* Static, human-readable text for a status code returned above (never NULL). */
const char *gemm_status_string(int status);

/*
 * Describe, without launching anything, the kernel variant the library picks
 * for a call with these arguments: writes a NUL-terminated text such as
 * "f32 mfma 128x128x32 loads A:vec4 B:vec4 C:vec2" into buf (at most len
 * bytes, truncated if needed).  dtype: 0 = fp32, 1 = fp16, 2 = fp16 inputs
 * with an fp32 C (gemm_f16f32).  Pointers are only
 * inspected for alignment.  Returns the status gemm_f32 / gemm_f16 would
 * return for the argument checks (0 or -i); no HIP call is made.
 */
int gemm_describe(int dtype, int M, int N, int K, float alpha,
                  const void *A, int lda, const void *B, int ldb,
                  float beta, const void *C, int ldc,
                  char *buf, int len);

/*
 * Diagnostic switch for tests: 0 = choose vector or scalar loads per operand
 * from alignment (the default); 1 = force scalar (element-wise) global loads
 * and stores for every operand.  Applies process-wide to later calls; not
 * meant for concurrent use with other threads issuing GEMMs.  Returns the
 * previous setting, or -1 for an unknown mode.
 */
int gemm_set_load_mode(int mode);

/*
 * Diagnostic switch for tests: 0 = choose the tile configuration from the
 * problem size (the default); 1, 2, 3, 4 = force the large, medium, small or
 * (fp32 only; fp16 uses its small one) tiny configuration; 5 = the medium
 * configuration with each K step's loads issued together rather than spread
 * (fp32 only; fp16 uses its medium one); 6 = the fp32 256 x 256 tile, and
 * for fp16 the large tile on 32x32x16 blocks (1 forces it on 16x16x32
 * blocks; the size-based choice takes either); 7 = the fp32 64 x 64 tile of
 * four 32 x 32 waves (fp16 uses its small one); 8 = the fp32 128 x 64 tile of
 * four 64 x 32 waves (fp16 uses its medium one); 9 = the fp32 64 x 64 tile of
 * four waves in 64-k steps through two LDS slots, 10 = the fp32 32 x 32 tile
 * of one wave in 64-k steps (fp16 uses its small one for both).
 * Process-wide,
 * like gemm_set_load_mode.  Returns the previous setting, or -1 for an
 * unknown value.
 */
int gemm_set_tile_config(int config);

/*
 * Diagnostic switch for tests: 0 = split K by problem size (the default);
 * 1 = never split; 2..64 = split K into that many chunks whenever K has that
 * many tile K steps (fewer otherwise).  Process-wide, like
 * gemm_set_load_mode.  Returns the previous setting, or -1 for an unknown
 * value.
 */
int gemm_set_split(int mode);

/*
 * Diagnostic switch for tests (fp32 calls): 0 = decide by problem size
 * whether the last, partly filled round of tiles runs as a split-K pass (the
 * default; see "Split K" above); 1 = never; 2..64 = split that round's tiles
 * into that many K chunks whenever the call has more tiles than CUs, is not
 * split as a whole, and the leftover tiles are at most half the CUs.
 * Process-wide, like gemm_set_load_mode.  Returns the previous setting, or -1
 * for an unknown value.
 */
int gemm_set_tail_split(int mode);

/*
 * Diagnostic switch for tests: 0 = copy A or B to 16-byte rows when their
 * rows do not allow 16-byte loads and the fp32 call is large enough (the
 * default; see "Operand copies" above); 1 = never copy; 2 = copy whenever
 * their rows do not allow 16-byte loads, whatever the size and type.  Copies are made
 * only where the workspace fits (gemm_set_workspace_limit) and never under
 * gemm_set_load_mode(1).  Process-wide, like gemm_set_load_mode.  Returns the
 * previous setting, or -1 for an unknown value.
 */
int gemm_set_pack(int mode);

/*
 * Diagnostic switch for tests (fp32): 0 = decide by problem size whether a
 * call runs Stream-K (the default; see "Stream-K" above); 1 = never; with
 * the 64x64 four-wave tile taken whole, or a tile forced by
 * gemm_set_tile_config (1, 5, 6 or 7), 2, 3, 4 = always, every tile's K
 * steps dealt out to 1, 2 or 3 workgroups per CU (in runs of at most one
 * tile's steps: more workgroups where the share would be longer); 5, 6 =
 * always, the whole rounds of one tile per CU first and the other tiles' K
 * steps dealt out to 1 or 2 more workgroups per CU (5 is the by-size
 * choice).  Calls whose workspace cannot be had run the plain launch.  Process-wide, like gemm_set_load_mode.
 * Returns the previous setting, or -1 for an unknown value.
 */
int gemm_set_stream_k(int mode);

/*
 * Cap on the workspace one call may take from the library's pool (operand
 * copies and split K), in bytes: -1 = no cap (the default), 0 = never use
 * workspace (every call runs unsplit, without copies), n > 0 = calls whose
 * copies and split need more than n bytes run without them (copies are
 * dropped first, then the split).
 * Process-wide, like gemm_set_load_mode; gemm_f32_noalloc ignores it.
 * Returns the previous setting, or -2 for a value below -1.
 */
long long gemm_set_workspace_limit(long long bytes);

/*
 * Matrix-core ceiling probe: a measurement aid, not a GEMM.  It bounds what
 * any GEMM kernel can reach on this part at the clock the part sustains
 * under matrix-core load (the power-aware comparison of the SGEMM summary's
 * discussion of tuning and power): one launch of 512 workgroups x 8 waves,
 * each wave running `iters` rounds of independent MFMAs over a 128 x 64
 * wave tile on operand registers loaded once (dtype 1: 32 of
 * v_mfma_f32_16x16x32_f16, fp16 operands; dtype 0: 8 of
 * v_mfma_f32_32x32x2_f32, fp32 operands: the large GEMM tiles' instructions),
 * with no memory traffic inside the loop.
 *   operands: DEVICE buffer of at least 65536 bytes holding fp16 (dtype 1)
 *             or fp32 (dtype 0) values; give it the distribution of the GEMM
 *             inputs being compared, since the MFMA power depends on the bits.
 *   out:      DEVICE buffer of at least 1 MiB; receives one float per thread
 *             (the sum of its accumulators), so that no MFMA is dead.
 *   flops:    HOST pointer; receives the launch's flop count
 *             (waves x iters x 2*128*64*k, k = 32 for fp16, 2 for fp32).
 * Enqueues one kernel on `stream` and returns 0, a positive hipError_t if the
 * launch fails, or -101 .. -107 for an invalid argument 1 .. 7 (checked in
 * order, before any HIP call).
 */
int gemm_probe_mfma(int dtype, int iters, const void *operands, size_t operand_bytes,
                    float *out, size_t out_bytes, double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_GEMM_H */
