// gemm_f32.hip -- fp32 GEMM on the gfx950 matrix cores.
//
// C := alpha*A*B + beta*C, row-major, fp32 in/out, fp32 accumulation with
// v_mfma_f32_32x32x2_f32.
//
// Structure (the tiling of the SGEMM summary's tiling section, mapped onto
// CDNA): each workgroup owns one BM x BN tile of C and walks K in steps of
// BK, staging the A (BM x BK) and B (BK x BN) tiles through double-buffered
// LDS; the next tiles' global loads are issued before the current tiles'
// MFMAs so their latency is hidden, with one barrier per K step.  Each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held in registers as FM x FN
// blocks of 32x32 accumulators.
//
// Operand layout.  For v_mfma_f32_32x32x2_f32 lane l supplies A(row l%32,
// k-slot l/32) and B(k-slot l/32, col l%32) and receives C(row
// 8*(r/4) + 4*(l/32) + r%4, col l%32) in accumulator register r.  Any
// permutation of k that A and B share leaves the sum unchanged, so:
//   * A is stored in LDS k-contiguous per row (padded by 4 floats so that 8
//     consecutive rows fall in distinct bank groups); one ds_read_b128 gives a
//     lane 4 consecutive k of its row, used by 4 successive MFMAs: lanes 0-31
//     take k = kk..kk+3, lanes 32-63 take k = kk+4..kk+7.
//   * B is stored as in memory (k rows, n contiguous).  Output columns are
//     interleaved inside a wave tile: MFMA block bj, lane column j holds
//     global column wn0 + FN*j + bj.  A lane therefore reads FN consecutive
//     floats of one B row with one LDS read, and in the epilogue writes FN
//     consecutive floats of each C row: 32 lanes cover 32*FN contiguous
//     floats, so stores are coalesced without a trip through LDS.
//
// Edges: tiles that cross M or N and the last, partial K step take masked
// loads that substitute 0 for every element outside the matrix (never a read
// of a pad element), and masked stores.  Interior tiles and full K steps run
// unmasked.  Alignment: A and B chunks are read with 128-bit loads when the
// leading dimension is a multiple of 4 and the base 16-byte aligned, else with
// 32-bit loads (the alignment gate of the SGEMM summary's texture-load
// variant).
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct F32Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NT = WAVES_M * WAVES_N * kWave;
  static constexpr int WTM = BM / WAVES_M;   // wave tile rows
  static constexpr int WTN = BN / WAVES_N;   // wave tile columns
  static constexpr int FM = WTM / 32;        // 32x32 blocks per wave (rows)
  static constexpr int FN = WTN / 32;        // 32x32 blocks per wave (cols) = C columns per lane
  static constexpr int SA = BK + 4;          // LDS row stride of the A tile (floats)
  static constexpr int SB = BN;              // LDS row stride of the B tile (floats)
  static constexpr int A_ELEMS = BM * SA;
  static constexpr int B_ELEMS = BK * SB;
  static constexpr int A_CHUNKS = BM * BK / 4 / NT;   // 4-float chunks per thread per K step
  static constexpr int B_CHUNKS = BK * BN / 4 / NT;
  static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * 4;
  static_assert(BM % (WAVES_M * 32) == 0 && BN % (WAVES_N * 32) == 0, "wave tiling");
  static_assert(BK % 8 == 0, "BK multiple of 8");
  static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "load split");
  static_assert(FN == 1 || FN == 2 || FN == 4, "FN");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int N> struct FVec;
template <> struct FVec<1> { typedef float type; };
template <> struct FVec<2> { typedef f32x2 type; };
template <> struct FVec<4> { typedef f32x4 type; };

// Global -> registers: the A tile rows m0.., columns k0..k0+BK-1.
template <class T, bool VEC, bool CHECK_M, bool CHECK_K>
__device__ __forceinline__ void load_a(const GemmParams &p, int m0, int k0,
                                       f32x4 (&ra)[T::A_CHUNKS]) {
  const float *A = static_cast<const float *>(p.A);
  constexpr int CPR = T::BK / 4;
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    const int row = c / CPR;
    const int kc = c % CPR;
    const int gr = m0 + row;
    const int gk = k0 + 4 * kc;
    const float *src = A + (size_t)gr * (size_t)p.lda + gk;
    const bool row_ok = !CHECK_M || gr < p.M;
    if (row_ok && (!CHECK_K || gk + 3 < p.K)) {
      if (VEC) {
        ra[i] = *reinterpret_cast<const f32x4 *>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ra[i][e] = src[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) ra[i][e] = (row_ok && gk + e < p.K) ? src[e] : 0.0f;
    }
  }
}

// Global -> registers: the B tile rows k0..k0+BK-1, columns n0...
template <class T, bool VEC, bool CHECK_N, bool CHECK_K>
__device__ __forceinline__ void load_b(const GemmParams &p, int n0, int k0,
                                       f32x4 (&rb)[T::B_CHUNKS]) {
  const float *B = static_cast<const float *>(p.B);
  constexpr int CPR = T::BN / 4;
#pragma unroll
  for (int i = 0; i < T::B_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    const int kr = c / CPR;
    const int nc = c % CPR;
    const int gk = k0 + kr;
    const int gn = n0 + 4 * nc;
    const float *src = B + (size_t)gk * (size_t)p.ldb + gn;
    const bool k_ok = !CHECK_K || gk < p.K;
    if (k_ok && (!CHECK_N || gn + 3 < p.N)) {
      if (VEC) {
        rb[i] = *reinterpret_cast<const f32x4 *>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[i][e] = src[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) rb[i][e] = (k_ok && gn + e < p.N) ? src[e] : 0.0f;
    }
  }
}

template <class T>
__device__ __forceinline__ void store_lds(float *As, float *Bs, const f32x4 (&ra)[T::A_CHUNKS],
                                          const f32x4 (&rb)[T::B_CHUNKS]) {
  constexpr int CPRA = T::BK / 4;
  constexpr int CPRB = T::BN / 4;
#pragma unroll
  for (int i = 0; i < T::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    *reinterpret_cast<f32x4 *>(&As[(c / CPRA) * T::SA + 4 * (c % CPRA)]) = ra[i];
  }
#pragma unroll
  for (int i = 0; i < T::B_CHUNKS; ++i) {
    const int c = threadIdx.x + i * T::NT;
    *reinterpret_cast<f32x4 *>(&Bs[(c / CPRB) * T::SB + 4 * (c % CPRB)]) = rb[i];
  }
}

// acc += A_tile(wave rows) * B_tile(wave cols) over the BK columns in LDS.
template <class T>
__device__ __forceinline__ void compute_tile(const float *As, const float *Bs, int wm0, int wn0,
                                             f32x16 (&acc)[T::FM][T::FN]) {
  typedef typename FVec<T::FN>::type BVec;
  const int lane = threadIdx.x % kWave;
  const int li = lane % 32;
  const int lh = lane / 32;
#pragma unroll
  for (int kk = 0; kk < T::BK; kk += 8) {
    f32x4 a[T::FM];
#pragma unroll
    for (int bi = 0; bi < T::FM; ++bi)
      a[bi] = *reinterpret_cast<const f32x4 *>(&As[(wm0 + 32 * bi + li) * T::SA + kk + 4 * lh]);
    BVec b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      b[s] = *reinterpret_cast<const BVec *>(&Bs[(kk + 4 * lh + s) * T::SB + wn0 + T::FN * li]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int bi = 0; bi < T::FM; ++bi) {
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj) {
          float bv;
          if constexpr (T::FN == 1) bv = b[s]; else bv = b[s][bj];
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bi][s], bv, acc[bi][bj], 0, 0, 0);
        }
      }
    }
  }
}

// alpha*acc + beta*C -> C for one wave tile whose origin is (r0, c0).
template <class T, bool VEC_C, bool CHECK>
__device__ __forceinline__ void epilogue(const GemmParams &p, int r0, int c0,
                                         const f32x16 (&acc)[T::FM][T::FN]) {
  typedef typename FVec<T::FN>::type CVec;
  float *C = static_cast<float *>(p.C);
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
      float *dst = C + (size_t)row * (size_t)p.ldc + col;
      float v[T::FN];
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj) v[bj] = alpha * acc[bi][bj][r];
      if (VEC_C && cols_ok) {
        CVec o;
        if (beta != 0.0f) {
          CVec cv = *reinterpret_cast<const CVec *>(dst);
          if constexpr (T::FN == 1) o = __builtin_fmaf(beta, cv, v[0]);
          else {
#pragma unroll
            for (int bj = 0; bj < T::FN; ++bj) o[bj] = __builtin_fmaf(beta, cv[bj], v[bj]);
          }
        } else {
          if constexpr (T::FN == 1) o = v[0];
          else {
#pragma unroll
            for (int bj = 0; bj < T::FN; ++bj) o[bj] = v[bj];
          }
        }
        *reinterpret_cast<CVec *>(dst) = o;
      } else {
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj) {
          if (CHECK && col + bj >= p.N) continue;
          float o = v[bj];
          if (beta != 0.0f) o = __builtin_fmaf(beta, dst[bj], o);
          dst[bj] = o;
        }
      }
    }
  }
}

template <class T, bool VA, bool VB, bool EDGE, bool CHECK_K>
__device__ __forceinline__ void load_tiles(const GemmParams &p, int m0, int n0, int k0,
                                           f32x4 (&ra)[T::A_CHUNKS], f32x4 (&rb)[T::B_CHUNKS]) {
  load_a<T, VA, EDGE, CHECK_K>(p, m0, k0, ra);
  load_b<T, VB, EDGE, CHECK_K>(p, n0, k0, rb);
}

template <class T, bool VA, bool VB, bool VC, bool EDGE>
__device__ __forceinline__ void mainloop(const GemmParams &p, int m0, int n0, float *lds) {
  float *As = lds;                   // [2][A_ELEMS]
  float *Bs = lds + 2 * T::A_ELEMS;  // [2][B_ELEMS]
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

  const int nk = (p.K + T::BK - 1) / T::BK;   // K >= 1 here
  const int nfull = p.K / T::BK;
  f32x4 ra[T::A_CHUNKS], rb[T::B_CHUNKS];

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
__global__ __launch_bounds__(T::NT) void sgemm_mfma(GemmParams p) {
  __shared__ __attribute__((aligned(16))) float lds[2 * (T::A_ELEMS + T::B_ELEMS)];
  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * T::BM;
  const int n0 = tn * T::BN;
  const bool edge = (m0 + T::BM > p.M) || (n0 + T::BN > p.N);
  if (edge) mainloop<T, VA, VB, VC, true>(p, m0, n0, lds);
  else mainloop<T, VA, VB, VC, false>(p, m0, n0, lds);
}

// ---------------------------------------------------------------- host side

// Tile configuration: BM, BN, BK, waves along M, waves along N, L2 group rows.
#ifndef DGEMM_F32_TILE
#define DGEMM_F32_TILE 128, 128, 32, 2, 2, 8
#endif
typedef F32Tile<DGEMM_F32_TILE> F32Main;
#define DGEMM_STR2(...) #__VA_ARGS__
#define DGEMM_STR(...) DGEMM_STR2(__VA_ARGS__)

static bool vec_ok(const void *p, int ld, int elems, int bytes_per_elem) {
  return (ld % elems) == 0 && aligned_to(p, (uintptr_t)elems * bytes_per_elem);
}

template <class T>
static Plan make_plan(const Call &c, const char *name) {
  Plan pl;
  pl.name = name;
  pl.bm = T::BM;
  pl.bn = T::BN;
  pl.bk = T::BK;
  pl.threads = T::NT;
  const bool va = !c.force_scalar && vec_ok(c.A, c.lda, 4, 4);
  const bool vb = !c.force_scalar && vec_ok(c.B, c.ldb, 4, 4);
  const bool vc = !c.force_scalar && T::FN > 1 && vec_ok(c.C, c.ldc, T::FN, 4);
  pl.vec_a = va ? 4 : 1;
  pl.vec_b = vb ? 4 : 1;
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
  hipLaunchKernelGGL((sgemm_mfma<T, VA, VB, VC>), dim3((unsigned)pl.blocks), dim3(T::NT), 0,
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

Plan plan_f32(const Call &c) {
  return make_plan<F32Main>(c, "f32 mfma32x32x2 tile " DGEMM_STR(DGEMM_F32_TILE));
}

hipError_t launch_f32(const Call &c) { return dispatch<F32Main>(c); }

}  // namespace dgemm
