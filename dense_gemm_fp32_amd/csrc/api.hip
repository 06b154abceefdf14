// api.hip -- the extern "C" entry points declared in include/gemm.h:
// argument checks, quick returns, variant choice and launch.
//
// Argument checks follow the BLAS convention (return -i for the first invalid
// argument i) and run before any HIP call.  The operation is
// C := alpha*A*B + beta*C on row-major matrices with leading dimensions (the
// SGEMM summary: definition and memory-layout section).
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/gemm.h"
#include "internal.hpp"

namespace {

std::atomic<int> g_load_mode{0};
std::atomic<int> g_tile_config{0};
std::atomic<int> g_split_mode{0};
std::atomic<int> g_tail_mode{0};
std::atomic<long long> g_ws_limit{-1};
std::atomic<int> g_pack_mode{0};
std::atomic<int> g_streamk_mode{0};

// Shared argument checks.  ta / tb: A is stored transposed (K x M, so its
// rows hold M elements) / B is (N x K, rows of K); otherwise A is M x K and B
// K x N.  Every matrix is row-major.
int check_args_t(bool ta, bool tb, int M, int N, int K, float alpha, const void *A, int lda,
                 const void *B, int ldb, float beta, const void *C, int ldc) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  const int row_a = ta ? M : K, row_b = tb ? K : N;
  if (lda < (row_a > 1 ? row_a : 1)) return -6;
  if (ldb < (row_b > 1 ? row_b : 1)) return -8;
  if (ldc < (N > 1 ? N : 1)) return -11;
  const bool empty = (M == 0 || N == 0);
  const bool reads_ab = !empty && K > 0 && alpha != 0.0f;
  if (reads_ab && A == nullptr) return -5;
  if (reads_ab && B == nullptr) return -7;
  const bool touches_c = !empty && !((alpha == 0.0f || K == 0) && beta == 1.0f);
  if (touches_c && C == nullptr) return -10;
  return 0;
}

int check_args(int M, int N, int K, float alpha, const void *A, int lda, const void *B, int ldb,
               float beta, const void *C, int ldc) {
  return check_args_t(false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
}

// The same checks for column-major operands (BLAS layout: X(i, j) at
// X[i + j*ldX]), with the argument indices of the column-major entry points.
int check_args_colmajor(int M, int N, int K, float alpha, const void *A, int lda, const void *B,
                        int ldb, float beta, const void *C, int ldc) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (lda < (M > 1 ? M : 1)) return -6;
  if (ldb < (K > 1 ? K : 1)) return -8;
  if (ldc < (M > 1 ? M : 1)) return -11;
  const bool empty = (M == 0 || N == 0);
  const bool reads_ab = !empty && K > 0 && alpha != 0.0f;
  if (reads_ab && A == nullptr) return -5;
  if (reads_ab && B == nullptr) return -7;
  const bool touches_c = !empty && !((alpha == 0.0f || K == 0) && beta == 1.0f);
  if (touches_c && C == nullptr) return -10;
  return 0;
}

enum class Route { kNothing, kScale, kGemm };

Route route(int M, int N, int K, float alpha, float beta) {
  if (M == 0 || N == 0) return Route::kNothing;
  if (alpha == 0.0f || K == 0) return beta == 1.0f ? Route::kNothing : Route::kScale;
  return Route::kGemm;
}

dgemm::Call make_call(int M, int N, int K, float alpha, const void *A, int lda, const void *B,
                      int ldb, float beta, void *C, int ldc, void *stream, bool out32 = false,
                      bool ta = false, bool tb = false) {
  dgemm::Call c;
  c.out32 = out32;
  c.ta = ta;
  c.tb = tb;
  c.M = M;
  c.N = N;
  c.K = K;
  c.alpha = alpha;
  c.beta = beta;
  c.A = A;
  c.lda = lda;
  c.B = B;
  c.ldb = ldb;
  c.C = C;
  c.ldc = ldc;
  c.force_scalar = g_load_mode.load(std::memory_order_relaxed) == 1;
  c.tile_config = g_tile_config.load(std::memory_order_relaxed);
  c.split_mode = g_split_mode.load(std::memory_order_relaxed);
  c.splits = 1;
  c.k_chunk = 0;
  c.split_stride = 0;
  c.tile_base = 0;
  c.tile_count = 0;
  c.c_tiles = false;
  c.tail_mode = g_tail_mode.load(std::memory_order_relaxed);
  c.ws_limit = g_ws_limit.load(std::memory_order_relaxed);
  c.ws_fixed = nullptr;
  c.ws_fixed_bytes = 0;
  c.pack_mode = g_pack_mode.load(std::memory_order_relaxed);
  c.streamk_mode = g_streamk_mode.load(std::memory_order_relaxed);
  c.stream = static_cast<hipStream_t>(stream);
  return c;
}

// One call of any type and layout: checks, quick returns, launch.
// kind: 0 = fp32, 1 = fp16 in and out, 2 = fp16 in, fp32 C.
int run_gemm(int kind, bool ta, bool tb, int M, int N, int K, float alpha, const void *A, int lda,
             const void *B, int ldb, float beta, void *C, int ldc, void *stream) {
  const int rc = check_args_t(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  hipError_t e = hipSuccess;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (route(M, N, K, alpha, beta)) {
    case Route::kNothing:
      return GEMM_SUCCESS;
    case Route::kScale:
      e = kind == 1 ? dgemm::launch_scale_f16(M, N, beta, static_cast<uint16_t *>(C), ldc, s)
                    : dgemm::launch_scale_f32(M, N, beta, static_cast<float *>(C), ldc, s);
      break;
    case Route::kGemm: {
      const dgemm::Call c = make_call(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                      kind == 2, ta, tb);
      e = kind == 0 ? dgemm::launch_f32(c) : dgemm::launch_f16(c);
      break;
    }
  }
  return e == hipSuccess ? GEMM_SUCCESS : (int)e;
}

}  // namespace

extern "C" {

int gemm_f32(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream) {
  return run_gemm(0, false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16(int M, int N, int K, float alpha, const gemm_half_t *A, int lda, const gemm_half_t *B,
             int ldb, float beta, gemm_half_t *C, int ldc, void *stream) {
  return run_gemm(1, false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16f32(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(2, false, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

// Transposed operands (row-major storage): the first letter gives A's
// operation, the second B's; "t": the operand is stored transposed (A as
// K x M, B as N x K) and multiplied as its transpose.
int gemm_f32_nt(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(0, false, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f32_tn(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(0, true, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f32_tt(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(0, true, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16_nt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc, void *stream) {
  return run_gemm(1, false, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16_tn(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc, void *stream) {
  return run_gemm(1, true, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16_tt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc, void *stream) {
  return run_gemm(1, true, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16f32_nt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(2, false, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16f32_tn(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(2, true, false, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16f32_tt(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                   const gemm_half_t *B, int ldb, float beta, float *C, int ldc, void *stream) {
  return run_gemm(2, true, true, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

// gemm_f32 for callers that cannot allocate: the same checks, plan and
// kernels, with the workspace (operand copies, split K) taken from the
// library's fixed scratch region instead of its memory pool.  A call whose plan needs more workspace
// than the region holds is refused before anything is enqueued.
int gemm_f32_noalloc(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                     int ldb, float beta, float *C, int ldc, void *stream) {
  const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  hipError_t e = hipSuccess;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (route(M, N, K, alpha, beta)) {
    case Route::kNothing:
      return GEMM_SUCCESS;
    case Route::kScale:
      e = dgemm::launch_scale_f32(M, N, beta, C, ldc, s);
      break;
    case Route::kGemm: {
      dgemm::Call c = make_call(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
      // The plan sees the region's size (copies of unaligned operands are
      // made only where they fit in it beside the split-K workspace); the
      // refusal comes before any HIP call.
      c.ws_fixed_bytes = dgemm::kScratchBytes;
      const dgemm::Plan p = dgemm::plan_f32(c);
      if (p.ws_bytes > dgemm::kScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
      e = dgemm::scratch_region(dgemm::stream_device(s), &c.ws_fixed);
      if (e != hipSuccess) return (int)e;
      e = dgemm::launch_f32(c);
      break;
    }
  }
  return e == hipSuccess ? GEMM_SUCCESS : (int)e;
}

int gemm_f32_valu(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                  int ldb, float beta, float *C, int ldc, void *stream) {
  const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  hipError_t e = hipSuccess;
  switch (route(M, N, K, alpha, beta)) {
    case Route::kNothing:
      return GEMM_SUCCESS;
    case Route::kScale:
      e = dgemm::launch_scale_f32(M, N, beta, C, ldc, static_cast<hipStream_t>(stream));
      break;
    case Route::kGemm:
      e = dgemm::launch_f32_valu(make_call(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream));
      break;
  }
  return e == hipSuccess ? GEMM_SUCCESS : (int)e;
}

// Column-major calls.  A column-major M x N matrix with leading dimension ld
// is, byte for byte, the row-major N x M matrix of its transpose with the same
// ld.  So C = A*B (all column-major) is the row-major product
// C^T = B^T * A^T: the row-major entry point with M and N exchanged and A and
// B exchanged, on the same buffers (the SGEMM summary's layout section:
// column-major use swaps A and B).  Arguments are checked first with the
// column-major rules and indices.
int gemm_f32_colmajor(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                      int ldb, float beta, float *C, int ldc, void *stream) {
  const int rc = check_args_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  return gemm_f32(N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

int gemm_f16_colmajor(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                      const gemm_half_t *B, int ldb, float beta, gemm_half_t *C, int ldc,
                      void *stream) {
  const int rc = check_args_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  return gemm_f16(N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

int gemm_f16f32_colmajor(int M, int N, int K, float alpha, const gemm_half_t *A, int lda,
                         const gemm_half_t *B, int ldb, float beta, float *C, int ldc,
                         void *stream) {
  const int rc = check_args_colmajor(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (rc != 0) return rc;
  return gemm_f16f32(N, M, K, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

const char *gemm_status_string(int status) {
  switch (status) {
    case 0: return "success";
    case -1: return "invalid argument 1: M < 0";
    case -2: return "invalid argument 2: N < 0";
    case -3: return "invalid argument 3: K < 0";
    case -5: return "invalid argument 5: A is NULL";
    case -6: return "invalid argument 6: lda < max(1, row length of A as stored: K, or M when A is stored transposed or column-major)";
    case -7: return "invalid argument 7: B is NULL";
    case -8: return "invalid argument 8: ldb < max(1, row length of B as stored: N, or K when B is stored transposed or column-major)";
    case -10: return "invalid argument 10: C is NULL";
    case -11: return "invalid argument 11: ldc < max(1, N) (row-major) or max(1, M) (column-major)";
    case GEMM_ERR_SCRATCH_LIMIT: return "gemm_f32_noalloc: the call's workspace (split K) would exceed the library's fixed scratch region (64 MiB); nothing was enqueued";
    case -101: return "invalid probe argument 1: dtype is not 0 (fp32) or 1 (fp16)";
    case -102: return "invalid probe argument 2: iters < 1";
    case -103: return "invalid probe argument 3: operands is NULL";
    case -104: return "invalid probe argument 4: operand buffer smaller than 65536 bytes";
    case -105: return "invalid probe argument 5: out is NULL";
    case -106: return "invalid probe argument 6: out buffer smaller than 1 MiB";
    case -107: return "invalid probe argument 7: flops is NULL";
    default: break;
  }
  if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
  return "unknown status";
}

int gemm_describe(int dtype, int M, int N, int K, float alpha, const void *A, int lda,
                  const void *B, int ldb, float beta, const void *C, int ldc, char *buf, int len) {
  const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  char text[256];
  if (rc != 0) {
    snprintf(text, sizeof text, "invalid: %s", gemm_status_string(rc));
  } else if (dtype < 0 || dtype > 2) {
    snprintf(text, sizeof text, "invalid: unknown dtype %d", dtype);
  } else {
    static const char *const kNames[3] = {"f32", "f16", "f16f32"};
    const char *dn = kNames[dtype];
    switch (route(M, N, K, alpha, beta)) {
      case Route::kNothing:
        snprintf(text, sizeof text, "%s no-op", dn);
        break;
      case Route::kScale:
        snprintf(text, sizeof text, "%s scale C := beta*C%s", dn,
                 beta == 0.0f ? " (zero fill, C not read)" : "");
        break;
      case Route::kGemm: {
        dgemm::Call c = make_call(M, N, K, alpha, A, lda, B, ldb, beta, const_cast<void *>(C), ldc,
                                  nullptr, dtype == 2);
        dgemm::Plan p = dtype ? dgemm::plan_f16(c) : dgemm::plan_f32(c);
        char split[48] = "";
        if (p.streamk && p.sk_whole > 0)
          snprintf(split, sizeof split, " stream-K after %lld whole tiles", p.sk_whole);
        else if (p.streamk) snprintf(split, sizeof split, " stream-K");
        else if (p.splits > 1) snprintf(split, sizeof split, " split-K %d", p.splits);
        else if (p.tail > 1) snprintf(split, sizeof split, " last round split-K %d", p.tail);
        char ws[48] = "";
        if (p.ws_bytes > 0) snprintf(ws, sizeof ws, " workspace %zu bytes", p.ws_bytes);
        const char *packed = p.packed_a ? (p.packed_b ? " copies A B" : " copies A")
                                        : (p.packed_b ? " copies B" : "");
        snprintf(text, sizeof text, "%s loads A:%s%d B:%s%d C:%s%d%s blocks %lld threads %d%s%s%s",
                 p.name, p.vec_a > 2 ? "vec" : (p.vec_a == 2 ? "pair" : "scalar"), p.vec_a,
                 p.vec_b > 2 ? "vec" : (p.vec_b == 2 ? "pair" : "scalar"), p.vec_b,
                 p.vec_c > 1 ? "vec" : "scalar", p.vec_c, packed, p.blocks, p.threads, split, ws,
                 beta == 0.0f ? " beta0 (C not read)" : "");
        break;
      }
    }
  }
  if (buf && len > 0) {
    strncpy(buf, text, (size_t)len - 1);
    buf[len - 1] = '\0';
  }
  return rc;
}

int gemm_probe_mfma(int dtype, int iters, const void *operands, size_t operand_bytes, float *out,
                    size_t out_bytes, double *flops, void *stream) {
  if (dtype != 0 && dtype != 1) return -101;
  if (iters < 1) return -102;
  if (operands == nullptr) return -103;
  if (operand_bytes < dgemm::probe_operand_bytes()) return -104;
  if (out == nullptr) return -105;
  if (out_bytes < dgemm::probe_out_bytes()) return -106;
  if (flops == nullptr) return -107;
  *flops = dgemm::probe_flops(dtype, iters);
  const hipError_t e = dgemm::launch_probe(dtype, iters, operands, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_SUCCESS : (int)e;
}

int gemm_set_load_mode(int mode) {
  if (mode != 0 && mode != 1) return -1;
  return g_load_mode.exchange(mode);
}

int gemm_set_split(int mode) {
  if (mode < 0 || mode > 64) return -1;
  return g_split_mode.exchange(mode);
}

int gemm_set_tail_split(int mode) {
  if (mode < 0 || mode > 64) return -1;
  return g_tail_mode.exchange(mode);
}

int gemm_set_tile_config(int config) {
  if (config < 0 || config > 10) return -1;
  return g_tile_config.exchange(config);
}

int gemm_set_pack(int mode) {
  if (mode < 0 || mode > 2) return -1;
  return g_pack_mode.exchange(mode);
}

int gemm_set_stream_k(int mode) {
  if (mode < 0 || mode > 6) return -1;
  return g_streamk_mode.exchange(mode);
}

long long gemm_set_workspace_limit(long long bytes) {
  if (bytes < -1) return -2;
  return g_ws_limit.exchange(bytes);
}

}  // extern "C"
