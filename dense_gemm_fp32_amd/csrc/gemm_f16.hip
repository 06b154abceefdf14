// gemm_f16.hip -- fp16-in / fp16-out GEMM with fp32 accumulation on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_f16).
//
// C := alpha*A*B + beta*C with A, B, C in binary16.  Products of halves are
// exact in fp32 and are accumulated in fp32; alpha*acc + beta*C is formed in
// fp32 and rounded once to half, round-to-nearest-even (the fp16 GEMM of the
// "LeetGPU GEMM T4" page: fp32 accumulators, one conversion at the end).
//
// Structure: the same double-buffered LDS K loop as the fp32 kernel (one
// barrier per K step, next tiles' global loads in flight during the MFMAs).
//
// Operand layout.  For v_mfma_f32_32x32x16_f16 lane l supplies 8 halves of
// A row l%32 and 8 halves of B column l%32 for the same k-slot group l/32, so
// both operands must be k-contiguous per lane:
//   * A tile in LDS: [BM rows][BK k] (+8 halves of row padding), copied
//     straight from memory with 128-bit loads.
//   * B tile in LDS: transposed to [BN columns][BK k].  Each thread loads a
//     4 (k) x 8 (n) block of B with four 128-bit loads, transposes it in
//     registers, and writes eight 4-half (64-bit) runs along k.
//   * Output columns are interleaved inside a wave tile (block bj, lane
//     column j holds wave column FN*j + bj), so each lane stores FN adjacent
//     halves of a C row and 32 lanes cover a contiguous run.  The transposed
//     B store places column FN*j + bj at LDS row 32*bj + j, so the MFMA reads
//     stay on consecutive LDS rows.
//
// Edges and alignment as in the fp32 kernel: masked loads that substitute 0
// outside the matrix on the edge tiles and the last K step, 128-bit loads only
// when the leading dimension is a multiple of 8 halves and the base 16-byte
// aligned, element-wise loads otherwise.
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct F16Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NT = WAVES_M * WAVES_N * kWave;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
  static constexpr int SA = BK + 8;            // LDS row stride of A (halves)
  static constexpr int SB = BK + 8;            // LDS row stride of B^T (halves)
  static constexpr int A_ELEMS = BM * SA;
  static constexpr int B_ELEMS = BN * SB;
  static constexpr int A_CHUNKS = BM * BK / 8 / NT;        // 8-half chunks per thread
  static constexpr int B_BLOCKS = (BK / 4) * (BN / 8) / NT;  // 4x8 blocks per thread
  static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * 2;
  static_assert(BM % (WAVES_M * 32) == 0 && BN % (WAVES_N * 32) == 0, "wave tiling");
  static_assert(BK % 16 == 0, "BK multiple of 16");
  static_assert((BM * BK / 8) % NT == 0, "A load split");
  static_assert(((BK / 4) * (BN / 8)) % NT == 0, "B load split");
  static_assert(FN == 1 || FN == 2 || FN == 4, "FN");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// 8 halves from global memory, element-wise or as one 128-bit load.
template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t *src) {
  if (VEC) return *reinterpret_cast<const u32x4 *>(src);
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (uint32_t)src[2 * e] | ((uint32_t)src[2 * e + 1] << 16);
  return v;
}

// 8 halves with per-element predicate ok(e); 0 where it fails.
template <class Ok>
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *src, Ok ok) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = ok(2 * e) ? (uint32_t)src[2 * e] : 0u;
    const uint32_t hi = ok(2 * e + 1) ? (uint32_t)src[2 * e + 1] : 0u;
    v[e] = lo | (hi << 16);
  }
  return v;
}

template <class T, bool VEC, bool CHECK_M, bool CHECK_K>
__device__ __forceinline__ void load_a(const GemmParams &p, int m0, int k0,
                                       u32x4 (&ra)[T::A_CHUNKS]) {
  const uint16_t *A = static_cast<const uint16_t *>(p.A);
  constexpr int CPR = T::BK / 8;
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    const int row = c / CPR;
    const int kc = c % CPR;
    const int gr = m0 + row;
    const int gk = k0 + 8 * kc;
    const uint16_t *src = A + (size_t)gr * (size_t)p.lda + gk;
    const bool row_ok = !CHECK_M || gr < p.M;
    if (row_ok && (!CHECK_K || gk + 7 < p.K)) {
      ra[i] = load8<VEC>(src);
    } else {
      const int K = p.K;
      ra[i] = load8_masked(src, [&](int e) { return row_ok && gk + e < K; });
    }
  }
}

// B block b of this thread: k rows 4*kg..4*kg+3 of the tile, columns 8*ng..8*ng+7.
template <class T>
__device__ __forceinline__ void b_block_coords(int i, int &kg, int &ng) {
  constexpr int KG = T::BK / 4;
  const int blk = threadIdx.x + i * T::NT;
  kg = blk % KG;
  ng = blk / KG;
}

template <class T, bool VEC, bool CHECK_N, bool CHECK_K>
__device__ __forceinline__ void load_b(const GemmParams &p, int n0, int k0,
                                       u32x4 (&rb)[T::B_BLOCKS][4]) {
  const uint16_t *B = static_cast<const uint16_t *>(p.B);
#pragma unroll
  for (int i = 0; i < T::B_BLOCKS; ++i) {
    int kg, ng;
    b_block_coords<T>(i, kg, ng);
    const int gn = n0 + 8 * ng;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gk = k0 + 4 * kg + r;
      const uint16_t *src = B + (size_t)gk * (size_t)p.ldb + gn;
      const bool k_ok = !CHECK_K || gk < p.K;
      if (k_ok && (!CHECK_N || gn + 7 < p.N)) {
        rb[i][r] = load8<VEC>(src);
      } else {
        const int N = p.N;
        rb[i][r] = load8_masked(src, [&](int e) { return k_ok && gn + e < N; });
      }
    }
  }
}

// LDS row of B^T that holds tile column n (see the interleaving note above).
template <class T>
__device__ __forceinline__ int bt_row(int n) {
  const int w = n / T::WTN;
  const int c = n % T::WTN;
  return w * T::WTN + 32 * (c % T::FN) + c / T::FN;
}

template <class T>
__device__ __forceinline__ void store_lds(uint16_t *As, uint16_t *Bs, const u32x4 (&ra)[T::A_CHUNKS],
                                          const u32x4 (&rb)[T::B_BLOCKS][4]) {
  constexpr int CPR = T::BK / 8;
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    *reinterpret_cast<u32x4 *>(&As[(c / CPR) * T::SA + 8 * (c % CPR)]) = ra[i];
  }
#pragma unroll
  for (int i = 0; i < T::B_BLOCKS; ++i) {
    int kg, ng;
    b_block_coords<T>(i, kg, ng);
    // Transpose the 4 x 8 block: column c8 becomes the 4-half run
    // (B[k+0][c8], B[k+1][c8], B[k+2][c8], B[k+3][c8]).
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
      const int sh = 16 * (c8 % 2);
      const uint32_t h0 = (rb[i][0][c8 / 2] >> sh) & 0xffffu;
      const uint32_t h1 = (rb[i][1][c8 / 2] >> sh) & 0xffffu;
      const uint32_t h2 = (rb[i][2][c8 / 2] >> sh) & 0xffffu;
      const uint32_t h3 = (rb[i][3][c8 / 2] >> sh) & 0xffffu;
      u32x2 run;
      run[0] = h0 | (h1 << 16);
      run[1] = h2 | (h3 << 16);
      *reinterpret_cast<u32x2 *>(&Bs[bt_row<T>(8 * ng + c8) * T::SB + 4 * kg]) = run;
    }
  }
}

template <class T>
__device__ __forceinline__ void compute_tile(const uint16_t *As, const uint16_t *Bs, int wm0,
                                             int wn0, f32x16 (&acc)[T::FM][T::FN]) {
  const int lane = threadIdx.x % kWave;
  const int li = lane % 32;
  const int lh = lane / 32;
#pragma unroll
  for (int kk = 0; kk < T::BK; kk += 16) {
    f16x8 a[T::FM], b[T::FN];
#pragma unroll
    for (int bi = 0; bi < T::FM; ++bi)
      a[bi] = *reinterpret_cast<const f16x8 *>(&As[(wm0 + 32 * bi + li) * T::SA + kk + 8 * lh]);
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
      b[bj] = *reinterpret_cast<const f16x8 *>(&Bs[(wn0 + 32 * bj + li) * T::SB + kk + 8 * lh]);
#pragma unroll
    for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
  }
}

template <class T, bool VEC_C, bool CHECK>
__device__ __forceinline__ void epilogue(const GemmParams &p, int r0, int c0,
                                         const f32x16 (&acc)[T::FM][T::FN]) {
  uint16_t *C = static_cast<uint16_t *>(p.C);
  const int lane = threadIdx.x % kWave;
  const int li = lane % 32;
  const int lh = lane / 32;
  const int col = c0 + T::FN * li;
  const float alpha = p.alpha, beta = p.beta;
  const bool cols_ok = !CHECK || col + T::FN - 1 < p.N;
#pragma unroll
  for (int bi = 0; bi < T::FM; ++bi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 32 * bi + 8 * (r / 4) + 4 * lh + (r % 4);
      if (CHECK && row >= p.M) continue;
      uint16_t *dst = C + (size_t)row * (size_t)p.ldc + col;
      if (VEC_C && cols_ok) {
        // FN adjacent halves: one 2*FN-byte access.
        uint16_t cin[T::FN];
        if (beta != 0.0f) {
          if constexpr (T::FN == 4) {
            const u32x2 w = *reinterpret_cast<const u32x2 *>(dst);
            cin[0] = w[0] & 0xffff; cin[1] = w[0] >> 16; cin[2] = w[1] & 0xffff; cin[3] = w[1] >> 16;
          } else if constexpr (T::FN == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(dst);
            cin[0] = w & 0xffff; cin[1] = w >> 16;
          } else {
            cin[0] = dst[0];
          }
        }
        uint16_t out[T::FN];
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj) {
          float v = alpha * acc[bi][bj][r];
          if (beta != 0.0f) v = __builtin_fmaf(beta, f16_bits_to_f32(cin[bj]), v);
          out[bj] = f32_to_f16_bits(v);
        }
        if constexpr (T::FN == 4) {
          u32x2 w;
          w[0] = (uint32_t)out[0] | ((uint32_t)out[1] << 16);
          w[1] = (uint32_t)out[2] | ((uint32_t)out[3] << 16);
          *reinterpret_cast<u32x2 *>(dst) = w;
        } else if constexpr (T::FN == 2) {
          *reinterpret_cast<uint32_t *>(dst) = (uint32_t)out[0] | ((uint32_t)out[1] << 16);
        } else {
          dst[0] = out[0];
        }
      } else {
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj) {
          if (CHECK && col + bj >= p.N) continue;
          float v = alpha * acc[bi][bj][r];
          if (beta != 0.0f) v = __builtin_fmaf(beta, f16_bits_to_f32(dst[bj]), v);
          dst[bj] = f32_to_f16_bits(v);
        }
      }
    }
  }
}

template <class T, bool VA, bool VB, bool EDGE, bool CHECK_K>
__device__ __forceinline__ void load_tiles(const GemmParams &p, int m0, int n0, int k0,
                                           u32x4 (&ra)[T::A_CHUNKS], u32x4 (&rb)[T::B_BLOCKS][4]) {
  load_a<T, VA, EDGE, CHECK_K>(p, m0, k0, ra);
  load_b<T, VB, EDGE, CHECK_K>(p, n0, k0, rb);
}

template <class T, bool VA, bool VB, bool VC, bool EDGE>
__device__ __forceinline__ void mainloop(const GemmParams &p, int m0, int n0, uint16_t *lds) {
  uint16_t *As = lds;
  uint16_t *Bs = lds + 2 * T::A_ELEMS;
  const int wave = threadIdx.x / kWave;
  const int wm0 = (wave / T::WAVES_N) * T::WTM;
  const int wn0 = (wave % T::WAVES_N) * T::WTN;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;

  const int nk = (p.K + T::BK - 1) / T::BK;
  const int nfull = p.K / T::BK;
  u32x4 ra[T::A_CHUNKS];
  u32x4 rb[T::B_BLOCKS][4];

  if (nfull > 0) load_tiles<T, VA, VB, EDGE, false>(p, m0, n0, 0, ra, rb);
  else load_tiles<T, VA, VB, EDGE, true>(p, m0, n0, 0, ra, rb);
  store_lds<T>(As, Bs, ra, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k1 = (kt + 1) * T::BK;
      if (kt + 1 < nfull) load_tiles<T, VA, VB, EDGE, false>(p, m0, n0, k1, ra, rb);
      else load_tiles<T, VA, VB, EDGE, true>(p, m0, n0, k1, ra, rb);
    }
    compute_tile<T>(As + cur * T::A_ELEMS, Bs + cur * T::B_ELEMS, wm0, wn0, acc);
    if (more) store_lds<T>(As + (cur ^ 1) * T::A_ELEMS, Bs + (cur ^ 1) * T::B_ELEMS, ra, rb);
    __syncthreads();
  }

  epilogue<T, VC, EDGE>(p, m0 + wm0, n0 + wn0, acc);
}

template <class T, bool VA, bool VB, bool VC>
__global__ __launch_bounds__(T::NT) void hgemm_mfma(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (T::A_ELEMS + T::B_ELEMS)];
  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * T::BM;
  const int n0 = tn * T::BN;
  const bool edge = (m0 + T::BM > p.M) || (n0 + T::BN > p.N);
  if (edge) mainloop<T, VA, VB, VC, true>(p, m0, n0, lds);
  else mainloop<T, VA, VB, VC, false>(p, m0, n0, lds);
}

// ---------------------------------------------------------------- host side

typedef F16Tile<256, 256, 32, 2, 2, 4> F16Main;

static bool vec_ok(const void *p, int ld, int elems) {
  return (ld % elems) == 0 && aligned_to(p, (uintptr_t)elems * 2);
}

template <class T>
static Plan make_plan(const Call &c, const char *name) {
  Plan pl;
  pl.name = name;
  pl.bm = T::BM;
  pl.bn = T::BN;
  pl.bk = T::BK;
  pl.threads = T::NT;
  const bool va = !c.force_scalar && vec_ok(c.A, c.lda, 8);
  const bool vb = !c.force_scalar && vec_ok(c.B, c.ldb, 8);
  const bool vc = !c.force_scalar && T::FN > 1 && vec_ok(c.C, c.ldc, T::FN);
  pl.vec_a = va ? 8 : 1;
  pl.vec_b = vb ? 8 : 1;
  pl.vec_c = vc ? T::FN : 1;
  const long long tm = (c.M + T::BM - 1) / T::BM;
  const long long tn = (c.N + T::BN - 1) / T::BN;
  pl.blocks = tm * tn;
  return pl;
}

template <class T, bool VA, bool VB, bool VC>
static hipError_t launch_variant(const Call &c, const Plan &pl) {
  GemmParams p;
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
  p.tiles_m = (c.M + T::BM - 1) / T::BM;
  p.tiles_n = (c.N + T::BN - 1) / T::BN;
  p.group_m = T::GROUP_M;
  hipLaunchKernelGGL((hgemm_mfma<T, VA, VB, VC>), dim3((unsigned)pl.blocks), dim3(T::NT), 0,
                     c.stream, p);
  return hipGetLastError();
}

template <class T>
static hipError_t dispatch(const Call &c) {
  const Plan pl = make_plan<T>(c, "");
  if (pl.blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int key = (pl.vec_a > 1 ? 4 : 0) | (pl.vec_b > 1 ? 2 : 0) | (pl.vec_c > 1 ? 1 : 0);
  switch (key) {
    case 0: return launch_variant<T, false, false, false>(c, pl);
    case 1: return launch_variant<T, false, false, true>(c, pl);
    case 2: return launch_variant<T, false, true, false>(c, pl);
    case 3: return launch_variant<T, false, true, true>(c, pl);
    case 4: return launch_variant<T, true, false, false>(c, pl);
    case 5: return launch_variant<T, true, false, true>(c, pl);
    case 6: return launch_variant<T, true, true, false>(c, pl);
    default: return launch_variant<T, true, true, true>(c, pl);
  }
}

Plan plan_f16(const Call &c) {
  return make_plan<F16Main>(c, "f16 mfma32x32x16 256x256x32 waves2x2");
}

hipError_t launch_f16(const Call &c) { return dispatch<F16Main>(c); }

}  // namespace dgemm
