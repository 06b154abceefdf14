// gemm_valu.hip -- fp32 GEMM on the vector ALUs, without the matrix cores.
//
// The SIMT design of the pages' SGEMM kernels, kept as the ablation against
// the MFMA path: C tiles staged through shared memory and register blocking
// per thread ("From 306 ms to 86 ms", register blocking: each thread owns a
// small block of C so that every value read from shared memory feeds several
// multiplies; the SGEMM summary's tiling section: block tiles, thread tiles of
// 8 x 8 outputs, A stored transposed in shared memory, double buffering).
//
// Here on gfx950: a 256-thread workgroup owns a 128 x 128 tile of C and walks
// K in steps of 16 through two LDS buffers.  Thread (ty, tx) of a 16 x 16
// grid holds an 8 x 8 block of C in registers: rows 4ty..4ty+3 and
// 64+4ty..64+4ty+3, columns 4tx..4tx+3 and 64+4tx..64+4tx+3, so each of its
// per-k reads is a 16-byte LDS read that lanes of equal ty share (broadcast)
// or that 16 lanes cover contiguously (conflict-free).  A is stored k-major
// ([k][m], rows padded by 4 floats, which puts the transposed 4-byte stores of
// a wave in 64 distinct banks), B as in memory ([k][n], padded alike).  Per k
// a thread issues 64 fp32 FMAs on the vector ALU (v_fmac_f32; the build
// excludes the packed two-wide form).  The ceiling is the fp32 vector peak,
// 157.3 TFLOP/s (256 CUs x 4 SIMDs x 64 flops per clock x 2.4 GHz), the same
// figure as the matrix cores' fp32 peak; this kernel measures ~82 at 4096^3.
//
// The next K step's tile is loaded into registers while the current one is
// multiplied and stored to the other buffer afterwards; one barrier per step.
// Loads are 16-byte vectors for interior tiles of aligned calls and masked
// element loads (0 outside the matrix) otherwise; stores are masked at the
// edges.  C := alpha*acc + beta*C in fp32; C is read only when beta != 0.
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

namespace {

constexpr int VBM = 128, VBN = 128, VBK = 16;
constexpr int VT = 256;
constexpr int VPAD = 4;
constexpr int ROWA = VBM + VPAD;   // floats per k row of the A buffer
constexpr int ROWB = VBN + VPAD;

struct ValuTile {
  f32x4 a[2];   // this thread's two 4-element chunks of the A tile (rows r, r+64)
  f32x4 b[2];   // ... of the B tile (k rows kr, kr+8)
};

// Thread t loads A rows t/4 and t/4 + 64, k columns 4*(t%4)..+3, and B k rows
// t/32 and t/32 + 8, columns 4*(t%32)..+3.
template <bool VEC>
__device__ __forceinline__ void valu_load(const GemmParams &p, int m0, int n0, int k0, bool interior,
                                          ValuTile &t) {
  const float *A = static_cast<const float *>(p.A);
  const float *B = static_cast<const float *>(p.B);
  const int tid = threadIdx.x;
  const int ar = tid / 4, ak = 4 * (tid % 4);
  const int bk = tid / 32, bn = 4 * (tid % 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int gr = m0 + ar + 64 * h, gk = k0 + ak;
    const float *src = A + (size_t)gr * (size_t)p.lda + gk;
    if (VEC && interior) {
      t.a[h] = *reinterpret_cast<const f32x4 *>(src);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) t.a[h][e] = (gr < p.M && gk + e < p.K) ? src[e] : 0.0f;
    }
    const int gkb = k0 + bk + 8 * h, gn = n0 + bn;
    const float *bsrc = B + (size_t)gkb * (size_t)p.ldb + gn;
    if (VEC && interior) {
      t.b[h] = *reinterpret_cast<const f32x4 *>(bsrc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) t.b[h][e] = (gkb < p.K && gn + e < p.N) ? bsrc[e] : 0.0f;
    }
  }
}

__device__ __forceinline__ void valu_store(const ValuTile &t, float *As, float *Bs) {
  const int tid = threadIdx.x;
  const int ar = tid / 4, ak = 4 * (tid % 4);
  const int bk = tid / 32, bn = 4 * (tid % 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 4; ++e) As[(ak + e) * ROWA + ar + 64 * h] = t.a[h][e];
    *reinterpret_cast<f32x4 *>(&Bs[(bk + 8 * h) * ROWB + bn]) = t.b[h];
  }
}

template <bool VEC_AB, bool VEC_C>
__global__ __launch_bounds__(VT) __attribute__((amdgpu_waves_per_eu(4))) void sgemm_valu(GemmParams p) {
  __shared__ __attribute__((aligned(16))) float As[2][VBK * ROWA];
  __shared__ __attribute__((aligned(16))) float Bs[2][VBK * ROWB];
  lds_poison(As, sizeof(As));
  lds_poison(Bs, sizeof(Bs));
  int tm, tn, split;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
  const int m0 = tm * VBM, n0 = tn * VBN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const bool rows_in = m0 + VBM <= p.M, cols_in = n0 + VBN <= p.N;

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  const int nk = (p.K + VBK - 1) / VBK;
  ValuTile t;
  valu_load<VEC_AB>(p, m0, n0, 0, rows_in && cols_in && VBK <= p.K, t);
  valu_store(t, As[0], Bs[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k1 = (kt + 1) * VBK;
      valu_load<VEC_AB>(p, m0, n0, k1, rows_in && cols_in && k1 + VBK <= p.K, t);
    }
    const float *as = As[cur];
    const float *bs = Bs[cur];
    // Unrolled by 4, not 16: fully unrolled, the compiler hoists all 64 LDS
    // reads of the step and needs ~370 VGPRs (one wave per SIMD).
#pragma unroll 4
    for (int k = 0; k < VBK; ++k) {
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&as[k * ROWA + 4 * ty]);
      const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&as[k * ROWA + 64 + 4 * ty]);
      const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&bs[k * ROWB + 4 * tx]);
      const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&bs[k * ROWB + 64 + 4 * tx]);
      float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (more) {
      // The other buffer was last read in step kt-1, before this step's
      // barrier (or never, at kt = 0).
      valu_store(t, As[cur ^ 1], Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  float *C = static_cast<float *>(p.C);
  const float alpha = p.alpha, beta = p.beta;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
    if (row >= p.M) continue;
#pragma unroll
    for (int hj = 0; hj < 2; ++hj) {
      const int col = n0 + 64 * hj + 4 * tx;
      float *dst = C + (size_t)row * (size_t)p.ldc + col;
      if (VEC_C && col + 3 < p.N) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = alpha * acc[i][4 * hj + e];
        if (beta != 0.0f) {
          const f32x4 c = *reinterpret_cast<const f32x4 *>(dst);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(beta, c[e], o[e]);
        }
        *reinterpret_cast<f32x4 *>(dst) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e >= p.N) continue;
          float o = alpha * acc[i][4 * hj + e];
          if (beta != 0.0f) o = __builtin_fmaf(beta, dst[e], o);
          dst[e] = o;
        }
      }
    }
  }
}

template <bool VEC_AB, bool VEC_C>
hipError_t valu_launch(const Call &c, long long tiles, int tiles_m, int tiles_n) {
  GemmParams p = {};
  p.A = c.A;
  p.B = c.B;
  p.C = c.C;
  p.M = c.M;
  p.N = c.N;
  p.K = c.K;
  p.lda = c.lda;
  p.ldb = c.ldb;
  p.ldc = c.ldc;
  p.alpha = c.alpha;
  p.beta = c.beta;
  p.tiles_m = tiles_m;
  p.tiles_n = tiles_n;
  p.group_m = 8;
  p.splits = 1;
  hipLaunchKernelGGL((sgemm_valu<VEC_AB, VEC_C>), dim3((unsigned)tiles), dim3(VT), 0, c.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_f32_valu(const Call &c) {
  const int tiles_m = (c.M + VBM - 1) / VBM, tiles_n = (c.N + VBN - 1) / VBN;
  const long long tiles = (long long)tiles_m * tiles_n;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // 16-byte loads need every row start of A and B 16-byte aligned.
  const bool vab = !c.force_scalar && (c.lda % 4) == 0 && (c.ldb % 4) == 0 &&
                   aligned_to(c.A, 16) && aligned_to(c.B, 16);
  const bool vc = !c.force_scalar && (c.ldc % 4) == 0 && aligned_to(c.C, 16);
  if (vab) return vc ? valu_launch<true, true>(c, tiles, tiles_m, tiles_n)
                     : valu_launch<true, false>(c, tiles, tiles_m, tiles_n);
  return vc ? valu_launch<false, true>(c, tiles, tiles_m, tiles_n)
            : valu_launch<false, false>(c, tiles, tiles_m, tiles_n);
}

}  // namespace dgemm
