// gemm_f32.hip -- fp32 GEMM on the gfx950 matrix cores.
//
// C := alpha*A*B + beta*C, row-major, fp32 in/out, fp32 accumulation with
// v_mfma_f32_32x32x2_f32.
//
// Pipeline.  Each workgroup owns a BM x BN tile of C and walks K in steps of
// BK (the tiling of the SGEMM summary's tiling section) through STAGES LDS
// slots filled by direct global->LDS loads (buffer_load_dwordx4 ... lds, 1 KB
// of LDS per wave instruction, no registers in between, 32-bit per-lane
// offsets against a per-step buffer base).  Each wave waits on vmcnt for its
// own loads of a slot and a raw barrier publishes it, so the loads of later
// steps stay in flight while this step is multiplied (the summary's
// shared-memory double buffering, deepened).  The barrier for step kt+1 sits
// inside the last k group of step kt, after half of its MFMAs, so the barrier
// wait overlaps them; by then every wave has read all of step kt, so step
// kt's slot can take step kt+STAGES.  The multi-wave tiles spread that step's
// loads over the following k slots, one between each group of MFMAs
// (mainloop_spread32; with two slots over the first half of the next step):
// issued all at once they fill the load queue, and the wave that blocks on a
// full queue also stops issuing MFMAs.  The one-wave tiles, which share a CU
// with other workgroups, issue them together (mainloop_direct32).  Each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as FM x FN blocks of 32x32
// accumulators.  A launch may cover part of the tile order, and its split-K
// pass may write dense per-tile blocks (the last-round split; see
// launch_tail).
//
// Operand layout.  For v_mfma_f32_32x32x2_f32 lane l supplies A(row l%32,
// k-slot l/32) and B(k-slot l/32, col l%32) and receives C(row
// 8*(r/4) + 4*(l/32) + r%4, col l%32) in accumulator register r.  Any
// permutation of k that A and B share leaves the sum unchanged, so:
//   * A sits in LDS k-contiguous per row, 16-byte chunks XOR-swizzled by row
//     ((r/2)%8 for 128-byte rows: the 16 rows one 128-bit read pass touches
//     fall in 16 distinct bank groups of gfx950's 64 banks).  One
//     ds_read_b128 gives a lane 4 consecutive k of its row, used by 4
//     successive MFMAs: lanes 0-31 take k = 8g..8g+3, lanes 32-63
//     k = 8g+4..8g+7.
//   * B sits as in memory (k rows, n contiguous).  Output columns are
//     interleaved inside a wave tile (block bj, lane column j holds wave
//     column FN*j + bj), so a lane reads FN adjacent floats of one B row per
//     k, and in the epilogue writes FN adjacent floats of each C row: 32
//     lanes cover 32*FN contiguous floats, coalesced straight from registers.
//   * Stored transposed, an operand keeps its stored orientation in LDS
//     (FRegion): A as K x M is read one float per lane per k slot, B as
//     N x K with one ds_read_b128 of 4 k per block column (its LDS rows in
//     the interleaved column order).
//
// Edges.  Direct loads cannot substitute zeros, so they only read chunks that
// lie inside the matrix: rows of a k-major operand past its extent (M for A,
// N for B) are clamped to the last row (they only feed C rows or columns that
// are never stored); chunks of an index-major operand past its extent are
// clamped to the last chunk when the extent is a multiple of 4.  The partial K
// step (K % BK != 0) runs first through registers with per-element masks.  A
// workgroup whose tile crosses the extent of an index-major operand that is
// not a multiple of 4, and every workgroup of a call whose A or B is not
// 16-byte aligned (base or leading dimension; the alignment gate of the SGEMM
// summary's texture-load variant) or whose offsets would reach 2^30 elements
// (32-bit load offsets), uses a register-staged path with masked loads (0
// outside the matrix; pad elements are never read) into the same LDS layout.
// Stores are masked on edge tiles.
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, int GROUP_M_,
          bool SPREAD_ = false>
struct S32Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr bool SPREAD = SPREAD_;               // direct path: loads spread over the step
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int STAGES = STAGES_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * kWave;
  // Epilogue: load a block's 16 rows of C before storing any of them.  It
  // costs registers, which the multi-wave tiles that share their CU (loads
  // issued together) need for their occupancy; their neighbours hide the
  // epilogue's memory latency instead.
  static constexpr bool C_BATCH = SPREAD || NWAVES == 1;
  static constexpr int WTM = BM / WAVES_M;              // wave tile rows
  static constexpr int WTN = BN / WAVES_N;              // wave tile columns
  static constexpr int FM = WTM / 32;                   // 32x32 blocks per wave (rows)
  static constexpr int FN = WTN / 32;                   // ... (cols) = C columns per lane
  static constexpr int KG = BK / 8;                     // 8-k groups per K step
  static constexpr int A_BYTES = BM * BK * 4;           // a slot's A region
  static constexpr int B_BYTES = BK * BN * 4;           // ... and B region
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int QA = A_BYTES / 1024;             // 1 KB wave loads per A tile
  static constexpr int QB = B_BYTES / 1024;
  static constexpr int QA_W = QA / NWAVES;              // ... per wave
  static constexpr int QB_W = QB / NWAVES;
  static constexpr int LOADS = QA_W + QB_W;             // direct loads per wave per K step
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(BM % (WAVES_M * 32) == 0 && BN % (WAVES_N * 32) == 0, "wave tiling");
  static_assert(BK % 8 == 0 && KG >= 1, "BK multiple of 8");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "1 KB load granules");
  static_assert(QA % NWAVES == 0 && QB % NWAVES == 0, "loads split over waves");
  static_assert(FN == 1 || FN == 2 || FN == 4, "FN");
  static_assert(STAGES >= 2, "the pipeline needs two or more slots");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(3 * LOADS <= 63, "vmcnt range");
};

template <int N> struct FVec;
template <> struct FVec<1> { typedef float type; };
template <> struct FVec<2> { typedef f32x2 type; };
template <> struct FVec<4> { typedef f32x4 type; };

// Operand regions.  A slot holds an A region (BM indices m by BK k) and a B
// region (BN indices n by BK k).  An operand whose memory is k-contiguous (A
// as stored, or B stored transposed, N x K) sits k-contiguous in LDS too
// ("k-major": rows of 4*BK bytes, one per index, chunks XOR-swizzled by
// (r / (256/ROW)) % (ROW/16) so that the 16 rows one 128-bit read pass
// touches fall in 16 distinct bank groups).  An operand whose memory is
// index-contiguous (B as stored, or A stored transposed, K x M) sits as in
// memory ("index-major": rows of 4*EXT bytes, one per k).  Direct loads copy
// 16-byte chunks, so the LDS orientation follows the memory layout.
//   * An index-major A is read one float per lane per k: lanes 0-31 read 32
//     consecutive m of k row kr, lanes 32-63 of row kr+4.  With rows of 256
//     bytes or more, chunk bit 3 is XORed with bit 2 of the row so that the
//     two rows' 128-byte pieces fall in different halves of the bank window.
//   * A k-major B is read in the wave tiles' interleaved column order (lane
//     column j of block bj is wave column FN*j + bj, so that the epilogue
//     writes FN adjacent floats per lane).  Its LDS rows therefore hold each
//     wave tile's columns in that order -- row 32*bj + j of a wave's WT rows
//     is column FN*j + bj -- so a 16-lane read pass touches 16 consecutive
//     rows.
template <int EXT, int BK, bool KMAJ, bool IDX_SWZ, int FN, int WT>
struct FRegion {
  static constexpr bool K_MAJOR = KMAJ;
  static constexpr int EXTENT = EXT;
  static constexpr int ROW = KMAJ ? 4 * BK : 4 * EXT;      // bytes per LDS row
  static constexpr int CH = ROW / 16;                       // 16-byte chunks per row
  static constexpr int RPW = ROW >= 256 ? 1 : 256 / ROW;    // rows per 256-byte window
  static_assert(!KMAJ || (32 % RPW == 0 && (32 / RPW) % CH == 0),
                "the swizzle repeats every 32 rows");
  static_assert(!KMAJ || FN == 1 || WT % (32 * FN) == 0, "wave tiles of whole blocks");

  __device__ static __forceinline__ int swz(int row) {
    if constexpr (KMAJ) return (row / RPW) % CH;
    else if constexpr (IDX_SWZ && CH >= 16) return 8 * ((row >> 2) & 1);
    else return 0;
  }

  // Index held by LDS row r of a k-major region.
  __device__ static __forceinline__ int index_of_row(int r) {
    if constexpr (KMAJ && FN > 1) {
      const int base = r / WT * WT, rin = r % WT;
      return base + FN * (rin % 32) + rin / 32;
    } else {
      return r;
    }
  }

  // Tile-relative index and k of the 4 elements behind 16-byte chunk
  // (q, lane) of the region (lane L of a 1 KB direct load writes bytes
  // q*1024 + 16L .. +15).
  __device__ static __forceinline__ void chunk(int q, int lane, int &idx, int &kk) {
    const int o = q * 1024 + 16 * lane;
    const int row = o / ROW;
    const int c = ((o % ROW) / 16) ^ swz(row);
    if constexpr (KMAJ) {
      idx = index_of_row(row);
      kk = 4 * c;
    } else {
      kk = row;
      idx = 4 * c;
    }
  }
};

// The two regions of tile T when A is stored transposed (TA) and/or B is
// (TB), and the LDS reads of one wave per 8-k group: k-major A one 128-bit
// read per block row, index-major A one float per block row and k; B as
// stored FN adjacent floats per k, k-major B one 128-bit read per block.
template <class T, bool TA_, bool TB_>
struct FLayout {
  static constexpr bool TA = TA_, TB = TB_;
  typedef FRegion<T::BM, T::BK, !TA_, true, 1, T::WTM> RA;
  typedef FRegion<T::BN, T::BK, TB_, false, T::FN, T::WTN> RB;
  static constexpr int NRA = TA_ ? 4 * T::FM : T::FM;
  static constexpr int NRB = TB_ ? T::FN : 4;
  static constexpr int NREAD = NRA + NRB;
};

// ---------------------------------------------------------------- direct loads

template <class T>
struct DirectAddr32 {
  uint32_t a[T::QA_W];   // byte offsets from the A tile origin of a K step
  uint32_t b[T::QB_W];   // ... and from the B tile origin
};

// Offset of the chunk at tile-relative (idx, kk) from the tile origin (index
// idx0, k k0).  Indices past the edge: k-major rows are clamped to the last
// row (they only feed rows or columns of C that are never stored);
// index-major chunks to the last whole chunk (ext % 4 == 0 on this path).
// The offsets do not change from step to step; each step only moves the
// buffer base.  They fit in 32 bits when EXT*ld (k-major) or BK*ld
// (index-major) is below 2^30 elements, which the kernel checks before
// taking this path.
template <class R>
__device__ __forceinline__ uint32_t direct_offset32(int idx, int kk, int idx0, int ext, int ld) {
  int g = idx0 + idx;
  if constexpr (R::K_MAJOR) {
    g = g < ext ? g : ext - 1;
    return 4u * (uint32_t)((g - idx0) * ld + kk);
  } else {
    g = g + 4 <= ext ? g : ext - 4;
    return 4u * (uint32_t)(kk * ld + (g - idx0));
  }
}

// First element of a K step's tile of an operand with leading dimension ld.
template <class R>
__device__ __forceinline__ const float *tile_base32(const void *X, int idx0, int k0, int ld) {
  const float *x = static_cast<const float *>(X);
  return R::K_MAJOR ? x + (size_t)idx0 * (size_t)ld + k0 : x + (size_t)k0 * (size_t)ld + idx0;
}

// The direct path's conditions for one operand: 32-bit offsets, and for an
// index-major operand whose tile crosses the edge, whole chunks up to it.
template <class R, int BK>
__device__ __forceinline__ bool direct_ok32(bool edge, int ext, int ld) {
  if constexpr (R::K_MAJOR) return (long long)R::EXTENT * ld < (1LL << 30);
  else return (!edge || (ext % 4) == 0) && (long long)BK * ld < (1LL << 30);
}

template <class T, class L>
__device__ __forceinline__ void direct_setup32(const GemmParams &p, int m0, int n0,
                                               DirectAddr32<T> &d) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j) {
    int idx, kk;
    L::RA::chunk(wave * T::QA_W + j, lane, idx, kk);
    d.a[j] = direct_offset32<typename L::RA>(idx, kk, m0, p.M, p.lda);
  }
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j) {
    int idx, kk;
    L::RB::chunk(wave * T::QB_W + j, lane, idx, kk);
    d.b[j] = direct_offset32<typename L::RB>(idx, kk, n0, p.N, p.ldb);
  }
}

template <class T, class L>
__device__ __forceinline__ void direct_issue32(const GemmParams &p, const DirectAddr32<T> &d,
                                               int m0, int n0, int k0, uint32_t slot_addr) {
  const int wave = wave_id();
  const BufRsrc ra = buffer_rsrc(tile_base32<typename L::RA>(p.A, m0, k0, p.lda));
  const BufRsrc rb = buffer_rsrc(tile_base32<typename L::RB>(p.B, n0, k0, p.ldb));
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j)
    buffer_load16(d.a[j], ra, slot_addr + (uint32_t)((wave * T::QA_W + j) * 1024));
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j)
    buffer_load16(d.b[j], rb, slot_addr + (uint32_t)(T::A_BYTES + (wave * T::QB_W + j) * 1024));
}

// ---------------------------------------------------------------- register-staged loads

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float *src) {
  if (VEC) return *reinterpret_cast<const f32x4 *>(src);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = src[e];
  return v;
}

// Four floats from an 8-byte aligned address as two 8-byte loads (rows whose
// leading dimension is even but not a multiple of 4: the SGEMM summary's
// memory-layout section ties 64-bit accesses to an even leading dimension).
__device__ __forceinline__ f32x4 load4_pairs(const float *src) {
  const f32x2 lo = *reinterpret_cast<const f32x2 *>(src);
  const f32x2 hi = *reinterpret_cast<const f32x2 *>(src + 2);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// A whole in-range chunk at width w (2 = 16 bytes, 1 = pairs, 0 = elements).
__device__ __forceinline__ f32x4 load4_width(const float *src, int w) {
  if (w == 2) return load4<true>(src);
  if (w == 1) return load4_pairs(src);
  return load4<false>(src);
}

template <class T>
struct RegTile32 {
  f32x4 a[T::QA_W];
  f32x4 b[T::QB_W];
};

// One chunk of an operand (tile origin idx0, k0) through registers, with 0
// for every element outside the matrix (index >= ext, k >= K).  `w`: the
// operand's load width (its rows start 16-byte aligned: a whole chunk is one
// load; 8-byte aligned: two; otherwise element by element).
template <class R>
__device__ __forceinline__ f32x4 staged_chunk32(const void *X, int ld, int idx0, int ext, int k0,
                                                int K, int idx, int kk, int w) {
  const int g = idx0 + idx, gk = k0 + kk;
  f32x4 v;
  if constexpr (R::K_MAJOR) {
    const float *src = static_cast<const float *>(X) + (size_t)g * (size_t)ld + gk;
    const bool ok = g < ext;
    if (ok && gk + 3 < K) return load4_width(src, w);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (ok && gk + e < K) ? src[e] : 0.0f;
  } else {
    const float *src = static_cast<const float *>(X) + (size_t)gk * (size_t)ld + g;
    const bool ok = gk < K;
    if (ok && g + 3 < ext) return load4_width(src, w);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (ok && g + e < ext) ? src[e] : 0.0f;
  }
  return v;
}

// The chunks the direct loads would fetch, through registers, with 0 for every
// element outside the matrix (rows >= M, columns >= N, k >= K).
template <class T, class L>
__device__ __forceinline__ void reg_load32(const GemmParams &p, int m0, int n0, int k0, int va,
                                           int vb, RegTile32<T> &t) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j) {
    int idx, kk;
    L::RA::chunk(wave * T::QA_W + j, lane, idx, kk);
    t.a[j] = staged_chunk32<typename L::RA>(p.A, p.lda, m0, p.M, k0, p.K, idx, kk, va);
  }
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j) {
    int idx, kk;
    L::RB::chunk(wave * T::QB_W + j, lane, idx, kk);
    t.b[j] = staged_chunk32<typename L::RB>(p.B, p.ldb, n0, p.N, k0, p.K, idx, kk, vb);
  }
}

template <class T>
__device__ __forceinline__ void reg_store32(const RegTile32<T> &t, char *slot) {
  const int wave = wave_id();
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j)
    *reinterpret_cast<f32x4 *>(slot + (wave * T::QA_W + j) * 1024 + 16 * lane) = t.a[j];
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j)
    *reinterpret_cast<f32x4 *>(slot + T::A_BYTES + (wave * T::QB_W + j) * 1024 + 16 * lane) =
        t.b[j];
}

// ---------------------------------------------------------------- fragments and MFMA

template <class T>
struct Frag32 {
  f32x4 a[T::FM];                       // 4 k of the lane's row in each block row
  typename FVec<T::FN>::type b[4];      // FN columns at each of the 4 k
};

// Per-lane LDS byte offsets of the fragments, relative to their region.
//   A k-major: block row 0 at k group g (block row bi adds 32*bi rows).
//   A index-major: block row bi at k 0 of the lane's half (k group g adds 8g
//     rows, k slot s adds s rows).
//   B as stored: k group 0, k slot 0 (k group g adds 8g rows, slot s adds s).
//   B k-major: block 0 at k group g (block bj adds 32*bj rows).
template <class T, class L>
struct FragAddr32 {
  int a[L::RA::K_MAJOR ? T::KG : T::FM];
  int b[L::RB::K_MAJOR ? T::KG : 1];
};

template <class T, class L>
__device__ __forceinline__ void frag_setup32(int wm0, int wn0, FragAddr32<T, L> &f) {
  typedef typename L::RA RA;
  typedef typename L::RB RB;
  const int lane = threadIdx.x % kWave;
  const int li = lane % 32, lh = lane / 32;
  if constexpr (RA::K_MAJOR) {
    const int r = wm0 + li;
    const int sa = RA::swz(r);
#pragma unroll
    for (int g = 0; g < T::KG; ++g) f.a[g] = r * RA::ROW + 16 * ((2 * g + lh) ^ sa);
  } else {
    // rows 8g + 4*lh + s all have the swizzle of row 4*lh
    const int sa = RA::swz(4 * lh);
#pragma unroll
    for (int bi = 0; bi < T::FM; ++bi) {
      const int m = wm0 + 32 * bi + li;
      f.a[bi] = 4 * lh * RA::ROW + 16 * ((m / 4) ^ sa) + 4 * (m % 4);
    }
  }
  if constexpr (RB::K_MAJOR) {
    const int r = wn0 + li;   // LDS row of lane column li of block 0
    const int sb = RB::swz(r);
#pragma unroll
    for (int g = 0; g < T::KG; ++g) f.b[g] = r * RB::ROW + 16 * ((2 * g + lh) ^ sb);
  } else {
    f.b[0] = 4 * lh * RB::ROW + 4 * (wn0 + T::FN * li);
  }
}

// LDS read number r (0 .. NREAD-1) of k group g: the B reads first (k order
// for B as stored, block order for a k-major B), then the A reads (block
// rows; for an index-major A, block row r/4 at k slot r%4).
template <class T, class L>
__device__ __forceinline__ void read_item32(int r, const char *slot, const FragAddr32<T, L> &f,
                                            int g, Frag32<T> &fr) {
  typedef typename L::RA RA;
  typedef typename L::RB RB;
  typedef typename FVec<T::FN>::type BVec;
  const char *rb = slot + T::A_BYTES;
  if (r < L::NRB) {
    if constexpr (RB::K_MAJOR) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(rb + f.b[g] + 32 * r * RB::ROW);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (T::FN == 1) fr.b[s] = v[s];
        else fr.b[s][r] = v[s];
      }
    } else {
      fr.b[r] = *reinterpret_cast<const BVec *>(rb + f.b[0] + (8 * g + r) * RB::ROW);
    }
  } else {
    const int q = r - L::NRB;
    if constexpr (RA::K_MAJOR)
      fr.a[q] = *reinterpret_cast<const f32x4 *>(slot + f.a[g] + 32 * q * RA::ROW);
    else
      fr.a[q / 4][q % 4] = *reinterpret_cast<const float *>(slot + f.a[q / 4] + (8 * g + q % 4) * RA::ROW);
  }
}

template <class T, class L>
__device__ __forceinline__ void frag_read32(const char *slot, const FragAddr32<T, L> &f, int g,
                                            Frag32<T> &fr) {
#pragma unroll
  for (int r = 0; r < L::NREAD; ++r) read_item32<T, L>(r, slot, f, g, fr);
}

// MFMAs of k slots [S0, S1) of one k group.
template <class T, int S0, int S1>
__device__ __forceinline__ void mfma_slots(const Frag32<T> &fr, f32x16 (&acc)[T::FM][T::FN]) {
#pragma unroll
  for (int s = S0; s < S1; ++s)
#pragma unroll
    for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj) {
        float bv;
        if constexpr (T::FN == 1) bv = fr.b[s]; else bv = fr.b[s][bj];
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.a[bi][s], bv, acc[bi][bj], 0, 0, 0);
      }
}

// Interleave pattern: one LDS read behind each of the first NR MFMAs.
template <int I, int NM, int NR>
__device__ __forceinline__ void interleave32_slot() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
    if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
    interleave32_slot<I + 1, NM, NR>();
  }
}

// All k groups of one K step from `slot`; fr[0] holds group 0 on entry.  The
// next group's fragments are read while the current group's MFMAs run.  In
// the last group, half of the MFMAs are issued, then `next()` publishes the
// following slot (its barrier wait overlaps those MFMAs), then group 0 of the
// following step is read from `next_slot` (a stale slot on the last step,
// never used) between the remaining MFMAs.
template <class T, class L, class Next>
__device__ __forceinline__ void kstep32(const char *slot, const char *next_slot,
                                        const FragAddr32<T, L> &fa, Frag32<T> (&fr)[2],
                                        f32x16 (&acc)[T::FM][T::FN], Next next) {
  constexpr int NREAD = L::NREAD;
  constexpr int NMF = 4 * T::FM * T::FN;
#pragma unroll
  for (int g = 0; g < T::KG; ++g) {
    if (g + 1 < T::KG) {
      frag_read32<T, L>(slot, fa, g + 1, fr[(g + 1) & 1]);
      mfma_slots<T, 0, 4>(fr[g & 1], acc);
      interleave32_slot<0, NMF, NREAD>();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      mfma_slots<T, 0, 2>(fr[g & 1], acc);
      __builtin_amdgcn_sched_barrier(0);
      next();
      frag_read32<T, L>(next_slot, fa, 0, fr[0]);
      mfma_slots<T, 2, 4>(fr[g & 1], acc);
      interleave32_slot<0, NMF / 2, NREAD>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------- main loops

template <class T, class L>
__device__ __forceinline__ void mainloop_direct32(const GemmParams &p, int m0, int n0, char *lds,
                                                  uint32_t lds_u32, int wm0, int wn0,
                                                  f32x16 (&acc)[T::FM][T::FN]) {
  const KSteps ks = make_steps(p.K, T::BK);
  DirectAddr32<T> da;
  direct_setup32<T, L>(p, m0, n0, da);
  FragAddr32<T, L> fa;
  frag_setup32<T, L>(wm0, wn0, fa);

  // Prologue: step 0 (masked, through registers, when it is the partial
  // step), then direct loads of steps 1 .. STAGES-1.
  if (ks.tail) {
    RegTile32<T> t;
    reg_load32<T, L>(p, m0, n0, ks.k0(0), 2, 2, t);
    reg_store32<T>(t, lds);
  } else {
    direct_issue32<T, L>(p, da, m0, n0, ks.k0(0), lds_u32);
  }
  int issued = 1;
#pragma unroll
  for (int j = 1; j < T::STAGES; ++j) {
    if (j < ks.nk) {
      direct_issue32<T, L>(p, da, m0, n0, ks.k0(j), lds_u32 + (uint32_t)(j * T::STAGE_BYTES));
      ++issued;
    }
  }
  wait_direct<T::LOADS>(issued - 1);
  lds_barrier();

  Frag32<T> fr[2];
  frag_read32<T, L>(lds, fa, 0, fr[0]);

  for (int kt = 0; kt < ks.nk; ++kt) {
    const int slot_no = kt % T::STAGES;
    const char *slot = lds + slot_no * T::STAGE_BYTES;
    const char *next_slot = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
    kstep32<T, L>(slot, next_slot, fa, fr, acc, [&]() {
      // Step kt+1 must have landed (steps issued after it may stay in
      // flight), and this wave's reads of step kt must be complete.
      wait_direct<T::LOADS>((issued - 1) - (kt + 1));
      lds_barrier();
      // Every wave has read all of step kt: its slot takes step kt+STAGES.
      const int nx = kt + T::STAGES;
      if (nx < ks.nk) {
        direct_issue32<T, L>(p, da, m0, n0, ks.k0(nx), lds_u32 + (uint32_t)(slot_no * T::STAGE_BYTES));
        ++issued;
      }
    });
  }
}

// One direct load (number j of this wave's LOADS per step) of the step whose
// buffer resources are (ra, rb) into the slot at `slot_addr`.
template <class T>
__device__ __forceinline__ void direct_one32(const DirectAddr32<T> &d, int j, BufRsrc ra,
                                             BufRsrc rb, uint32_t slot_addr, int wave) {
  if (j < T::QA_W)
    buffer_load16(d.a[j], ra, slot_addr + (uint32_t)((wave * T::QA_W + j) * 1024));
  else
    buffer_load16(d.b[j - T::QA_W], rb,
                  slot_addr + (uint32_t)(T::A_BYTES + (wave * T::QB_W + j - T::QA_W) * 1024));
}

// The step whose loads are in progress: its buffer resources and LDS slot.
struct Fill {
  BufRsrc ra, rb;
  uint32_t slot_addr;
  bool live;           // the step exists (index < nk)
};

template <class T, class L>
__device__ __forceinline__ Fill make_fill(const GemmParams &p, const KSteps &ks, int step, int m0,
                                          int n0, uint32_t slot_addr) {
  Fill f;
  f.live = step < ks.nk;
  f.slot_addr = slot_addr;
  const int k0 = f.live ? ks.k0(step) : 0;
  f.ra = buffer_rsrc(tile_base32<typename L::RA>(p.A, m0, k0, p.lda));
  f.rb = buffer_rsrc(tile_base32<typename L::RB>(p.B, n0, k0, p.ldb));
  return f;
}

// Direct-load pipeline with the loads spread out.  A step has NS = 4*KG k
// slots of FM*FN MFMAs each.  The barrier that publishes step kt+1 sits after
// k slot NS-3 of step kt (half of the last k group); once past it, every wave
// has read all of step kt, so step kt's slot takes step kt+STAGES.  Instead of
// issuing that step's LOADS loads at once -- which fills the load queue and
// holds up the issuing wave, and with it the MFMAs of its SIMD -- one load (or
// a few, evenly) follows each of the next NS k slots: slots NS-2 and NS-1 of
// step kt and slots 0 .. NS-3 of step kt+1.  A step's last load is thus issued
// just before the barrier of the step that follows the one that started it,
// and is needed STAGES-2 barriers later.  With two slots a load is needed at
// that very barrier, so the loads are spread over the first NS/2 gaps only:
// the last one then has half a step (thousands of MFMA cycles) to land.
template <class T, class L>
__device__ __forceinline__ void mainloop_spread32(const GemmParams &p, int m0, int n0, char *lds,
                                                  uint32_t lds_u32, int wm0, int wn0,
                                                  f32x16 (&acc)[T::FM][T::FN]) {
  static_assert(T::STAGES >= 2 && T::STAGES - 2 <= 3, "vmcnt steps");
  static_assert(T::KG % 2 == 0, "the last k group reads the next step's group 0 into fr[0]");
  constexpr int NS = 4 * T::KG;            // k slots per step
  constexpr int GAPS = T::STAGES >= 3 ? NS : NS / 2;   // gaps the loads are spread over
  constexpr int NL = T::LOADS;
  constexpr int NREAD = L::NREAD;          // LDS reads per k group
  constexpr int RPS = (NREAD + 3) / 4;     // reads placed after each k slot
  static_assert(2 * RPS <= 16, "reads per k slot");
  const KSteps ks = make_steps(p.K, T::BK);
  DirectAddr32<T> da;
  direct_setup32<T, L>(p, m0, n0, da);
  FragAddr32<T, L> fa;
  frag_setup32<T, L>(wm0, wn0, fa);
  const int wave = wave_id();

  if (ks.tail) {
    RegTile32<T> t;
    reg_load32<T, L>(p, m0, n0, ks.k0(0), 2, 2, t);
    reg_store32<T>(t, lds);
  } else {
    direct_issue32<T, L>(p, da, m0, n0, ks.k0(0), lds_u32);
  }
  int pro = 0;
#pragma unroll
  for (int j = 1; j < T::STAGES; ++j) {
    if (j < ks.nk) {
      direct_issue32<T, L>(p, da, m0, n0, ks.k0(j), lds_u32 + (uint32_t)(j * T::STAGE_BYTES));
      ++pro;
    }
  }
  wait_direct<NL>(pro);
  lds_barrier();

  Frag32<T> fr[2];
  frag_read32<T, L>(lds, fa, 0, fr[0]);
  // Before the first barrier nothing is being refilled.
  Fill fill = make_fill<T, L>(p, ks, ks.nk, m0, n0, 0);

  for (int kt = 0; kt < ks.nk; ++kt) {
    const int slot_no = kt % T::STAGES;
    const char *slot = lds + slot_no * T::STAGE_BYTES;
    const char *next_slot = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
#pragma unroll
    for (int g = 0; g < T::KG; ++g) {
      Frag32<T> &cur = fr[g & 1];
      Frag32<T> &nxt = fr[(g + 1) & 1];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int kslot = 4 * g + sl;
        if (kslot == NS - 2) {
          // Publish step kt+1: steps up to kt+STAGES-1 are fully issued.
          const int steps_after = (ks.nk < kt + T::STAGES ? ks.nk : kt + T::STAGES) - kt - 2;
          wait_direct<NL>(steps_after);
          lds_barrier();
          fill = make_fill<T, L>(p, ks, kt + T::STAGES, m0, n0,
                                 lds_u32 + (uint32_t)(slot_no * T::STAGE_BYTES));
        }
        // LDS reads for the next k group (or the next step's group 0), a
        // few after each k slot's MFMAs.
        const bool last = g + 1 == T::KG;
        if (!last || sl >= 2) {
          const int first = last ? 2 * RPS * (sl - 2) : RPS * sl;
          const int cnt = last ? 2 * RPS : RPS;
          const char *rs = last ? next_slot : slot;
          const int rg = last ? 0 : g + 1;
          // Reads in frag_read32's order (read_item32).
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = first + q;
            if (q < cnt && r < NREAD) read_item32<T, L>(r, rs, fa, rg, nxt);
          }
        }
#pragma unroll
        for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
          for (int bj = 0; bj < T::FN; ++bj) {
            float bv;
            if constexpr (T::FN == 1) bv = cur.b[sl]; else bv = cur.b[sl][bj];
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur.a[bi][sl], bv, acc[bi][bj], 0, 0, 0);
          }
        __builtin_amdgcn_sched_barrier(0);
        // Loads of the step being filled: gap number `gap` of NS since the
        // barrier that freed its slot.
        const int gap = kslot >= NS - 2 ? kslot - (NS - 2) : kslot + 2;
#pragma unroll
        for (int j = 0; j < NL; ++j)
          if ((j * GAPS) / NL == gap && fill.live) direct_one32<T>(da, j, fill.ra, fill.rb, fill.slot_addr, wave);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <class T, class L>
__device__ __forceinline__ void mainloop_staged32(const GemmParams &p, int m0, int n0, char *lds,
                                                  int wm0, int wn0, int va, int vb,
                                                  f32x16 (&acc)[T::FM][T::FN]) {
  const KSteps ks = make_steps(p.K, T::BK);
  FragAddr32<T, L> fa;
  frag_setup32<T, L>(wm0, wn0, fa);
  RegTile32<T> t;
  reg_load32<T, L>(p, m0, n0, ks.k0(0), va, vb, t);
  reg_store32<T>(t, lds);
  __syncthreads();
  Frag32<T> fr[2];
  frag_read32<T, L>(lds, fa, 0, fr[0]);
  for (int kt = 0; kt < ks.nk; ++kt) {
    const char *slot = lds + (kt % 2) * T::STAGE_BYTES;
    char *nslot = lds + ((kt + 1) % 2) * T::STAGE_BYTES;
    if (kt + 1 < ks.nk) reg_load32<T, L>(p, m0, n0, ks.k0(kt + 1), va, vb, t);
    // nslot was last read in step kt-1, before that step's barrier.  On the
    // last step the store repeats old data into a slot nobody reads again.
    kstep32<T, L>(slot, nslot, fa, fr, acc, [&]() {
      reg_store32<T>(t, nslot);
      __syncthreads();
    });
  }
}

// ---------------------------------------------------------------- epilogue

// alpha*acc + beta*C -> C for one wave tile whose origin is (r0, c0).
template <class T, bool VEC_C, bool CHECK>
__device__ __forceinline__ void epilogue32(const GemmParams &p, int r0, int c0,
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
    if constexpr (!VEC_C) {
      // Element-wise C (unaligned ldc or base): the C values of G rows are
      // loaded, masked, before the first of them is stored, so the rows wait
      // out one memory latency per group instead of one per row (a store to
      // C keeps a later load of C from moving above it).  G = 16 (the whole
      // block) where the tile's registers allow it, else 4.
      constexpr int G = T::C_BATCH ? 16 : 4;
#pragma unroll
      for (int g0 = 0; g0 < 16; g0 += G) {
        float cs[G][T::FN];
        if (beta != 0.0f) {
#pragma unroll
          for (int r = 0; r < G; ++r) {
            const int row = r0 + 32 * bi + 8 * ((g0 + r) / 4) + 4 * lh + ((g0 + r) % 4);
            const float *src = C + (size_t)row * (size_t)p.ldc + col;
#pragma unroll
            for (int bj = 0; bj < T::FN; ++bj)
              cs[r][bj] = (!CHECK || (row < p.M && col + bj < p.N)) ? src[bj] : 0.0f;
          }
        }
#pragma unroll
        for (int r = 0; r < G; ++r) {
          const int row = r0 + 32 * bi + 8 * ((g0 + r) / 4) + 4 * lh + ((g0 + r) % 4);
          if (CHECK && row >= p.M) continue;
          float *dst = C + (size_t)row * (size_t)p.ldc + col;
#pragma unroll
          for (int bj = 0; bj < T::FN; ++bj) {
            if (CHECK && col + bj >= p.N) continue;
            const float v = alpha * acc[bi][bj][g0 + r];
            dst[bj] = beta != 0.0f ? __builtin_fmaf(beta, cs[r][bj], v) : v;
          }
        }
      }
      continue;
    }
    // With C_BATCH the block's 16 rows of C are all loaded before the first
    // store: a load placed after a store to the same array cannot be moved
    // above it, so interleaved they wait out one memory latency per row.
    // (The lanes past an edge tile's last full column group load theirs
    // element by element as they store.)
    CVec cin[16];
    if (T::C_BATCH && VEC_C && cols_ok && beta != 0.0f) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + 32 * bi + 8 * (r / 4) + 4 * lh + (r % 4);
        if (!CHECK || row < p.M)
          cin[r] = *reinterpret_cast<const CVec *>(C + (size_t)row * (size_t)p.ldc + col);
      }
    }
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
          const CVec cv = T::C_BATCH ? cin[r] : *reinterpret_cast<const CVec *>(dst);
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

// The product of one C tile (origin m0, n0) over p's K range (p.A and p.B
// point at its first k) into acc: direct loads where the tile and its
// operands allow them, else the register-staged path.  Returns with every
// load complete.
template <class T, bool TA, bool TB>
__device__ __forceinline__ void tile_product(const GemmParams &p, int m0, int n0, char *lds,
                                             int wm0, int wn0, f32x16 (&acc)[T::FM][T::FN]) {
  typedef FLayout<T, TA, TB> L;
#pragma unroll
  for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;

  const bool m_edge = m0 + T::BM > p.M;
  const bool n_edge = n0 + T::BN > p.N;
  const int va = vec_width_a(p.vec_ab), vb = vec_width_b(p.vec_ab);
  const bool direct = va == 2 && vb == 2 && direct_ok32<typename L::RA, T::BK>(m_edge, p.M, p.lda) &&
                      direct_ok32<typename L::RB, T::BK>(n_edge, p.N, p.ldb);
  if (direct) {
    if constexpr (T::SPREAD) mainloop_spread32<T, L>(p, m0, n0, lds, lds_address(lds), wm0, wn0, acc);
    else mainloop_direct32<T, L>(p, m0, n0, lds, lds_address(lds), wm0, wn0, acc);
  } else {
    mainloop_staged32<T, L>(p, m0, n0, lds, wm0, wn0, va, vb, acc);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
}

// TA / TB: A is stored transposed (K x M, lda >= M) / B is (N x K, ldb >= K).
template <class T, bool TA, bool TB, bool VC>
__global__ __launch_bounds__(T::NT) void sgemm_mfma(GemmParams p) {
  typedef FLayout<T, TA, TB> L;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];
  lds_poison(lds, T::LDS_BYTES);
  int tm, tn, split, local;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m,
                p.tile_count > 0 ? p.tile_count : p.tiles_m * p.tiles_n, p.tile_base, tm, tn, split,
                local);
  select_split<float, float, TA, TB>(p, split);
  const int m0 = tm * T::BM;
  const int n0 = tn * T::BN;
  const int wave = wave_id();
  const int wm0 = (wave / T::WAVES_N) * T::WTM;
  const int wn0 = (wave % T::WAVES_N) * T::WTN;
  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;

  const bool m_edge = m0 + T::BM > p.M;
  const bool n_edge = n0 + T::BN > p.N;
  const int va = vec_width_a(p.vec_ab), vb = vec_width_b(p.vec_ab);
  const bool direct = va == 2 && vb == 2 && direct_ok32<typename L::RA, T::BK>(m_edge, p.M, p.lda) &&
                      direct_ok32<typename L::RB, T::BK>(n_edge, p.N, p.ldb);
  if (direct) {
    if constexpr (T::SPREAD) mainloop_spread32<T, L>(p, m0, n0, lds, lds_address(lds), wm0, wn0, acc);
    else mainloop_direct32<T, L>(p, m0, n0, lds, lds_address(lds), wm0, wn0, acc);
  } else {
    mainloop_staged32<T, L>(p, m0, n0, lds, wm0, wn0, va, vb, acc);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);

  if (p.c_tiles) {
    // Split-K pass over a run of tiles: this (split, tile)'s raw sums fill a
    // dense BM x BN block of the workspace (rows and columns past the matrix
    // included; the reduction ignores them).  alpha = 1, beta = 0 here.
    GemmParams q = p;
    q.C = static_cast<float *>(p.C) + ((size_t)split * (size_t)p.tile_count + (size_t)local) *
                                          (size_t)(T::BM * T::BN);
    q.ldc = T::BN;
    epilogue32<T, true, false>(q, wm0, wn0, acc);
    return;
  }
  const bool edge = n_edge || m_edge;
  if (edge) epilogue32<T, VC, true>(p, m0 + wm0, n0 + wn0, acc);
  else epilogue32<T, VC, false>(p, m0 + wm0, n0 + wn0, acc);
}

// Stream-K (the SGEMM summary's results section names it as the next step
// beyond fixed tiles), optionally behind whole tiles.  Workgroups with
// blockIdx.x < sk.dp each compute one of tiles 0 .. dp-1 whole, in the
// XCD-aware order of sgemm_mfma.  The K steps of the remaining tiles, tile
// after tile in the grouped order, are dealt out in equal runs of sk.iters to
// the other workgroups, so that every CU ends up with the same work whatever
// the tile count; dp is a whole number of rounds of one tile per CU, and the
// hardware hands out workgroups in blockIdx order, so each CU holds the same
// mix of whole-tile and Stream-K workgroups.  A run is at most one tile's K
// steps long, so it touches one tile or crosses into a second (two
// segments, written out rather than looped: a loop kept the load addresses
// of one segment live through the next, past the larger tiles' register
// budgets); a segment covering its tile whole is written to C as usual, and
// a part of a tile is written as raw fp32 sums to the workgroup's workspace
// slot: 2g for its first segment, 2g + 1 for its second, g the workgroup's
// position among the Stream-K workgroups in XCD-remapped order.
// The fix-up pass (launch_streamk_fixup) then sums each shared tile's slots
// in workgroup order -- ascending K -- and applies alpha and beta, so results
// do not depend on which workgroup finishes first.
template <class T, bool TA, bool TB, bool VC>
__global__ __launch_bounds__(T::NT) void sgemm_streamk(GemmParams p, StreamKRun sk) {
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];
  lds_poison(lds, T::LDS_BYTES);
  const int wave = wave_id();
  const int wm0 = (wave / T::WAVES_N) * T::WTM;
  const int wn0 = (wave % T::WAVES_N) * T::WTN;
  const int bid = blockIdx.x;
  if (bid < sk.dp) {
    int tm, tn;
    tile_coords(xcd_order(bid, sk.dp), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    f32x16 acc[T::FM][T::FN];
    tile_product<T, TA, TB>(p, m0, n0, lds, wm0, wn0, acc);
    const bool edge = n0 + T::BN > p.N || m0 + T::BM > p.M;
    if (edge) epilogue32<T, VC, true>(p, m0 + wm0, n0 + wn0, acc);
    else epilogue32<T, VC, false>(p, m0 + wm0, n0 + wn0, acc);
    return;
  }
  const int g = xcd_order(bid - sk.dp, (int)gridDim.x - sk.dp);
  const long long it_all = (long long)(sk.tiles - sk.dp) * sk.steps;
  long long it = (long long)g * sk.iters;
  const long long it1 = it + sk.iters < it_all ? it + sk.iters : it_all;
  auto segment = [&](bool first) {
    const int local = (int)(it / sk.steps);
    const int kb = (int)(it - (long long)local * sk.steps);
    const long long room = it1 - it;
    const int ke = room < (long long)(sk.steps - kb) ? kb + (int)room : sk.steps;
    int tm, tn;
    tile_coords(sk.dp + local, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int k_lo = kb * T::BK;
    const int k_hi = (long long)ke * T::BK < (long long)p.K ? ke * T::BK : p.K;
    GemmParams q = p;
    q.K = k_hi - k_lo;
    q.A = static_cast<const float *>(p.A) + (TA ? (size_t)k_lo * (size_t)p.lda : (size_t)k_lo);
    q.B = static_cast<const float *>(p.B) + (TB ? (size_t)k_lo : (size_t)k_lo * (size_t)p.ldb);
    f32x16 acc[T::FM][T::FN];
    tile_product<T, TA, TB>(q, m0, n0, lds, wm0, wn0, acc);
    if (kb == 0 && ke == sk.steps) {
      const bool edge = n0 + T::BN > p.N || m0 + T::BM > p.M;
      if (edge) epilogue32<T, VC, true>(p, m0 + wm0, n0 + wn0, acc);
      else epilogue32<T, VC, false>(p, m0 + wm0, n0 + wn0, acc);
    } else {
      GemmParams w = p;
      w.C = sk.W + (size_t)(2 * g + (first ? 0 : 1)) * (size_t)(T::BM * T::BN);
      w.ldc = T::BN;
      w.alpha = 1.0f;
      w.beta = 0.0f;
      epilogue32<T, true, false>(w, wm0, wn0, acc);
    }
    it += ke - kb;
  };
  segment(true);
  if (it < it1) {
    __syncthreads();
    segment(false);
  }
}

// ---------------------------------------------------------------- host side

// Tile configurations (BM, BN, BK, waves along M, waves along N, LDS slots,
// L2 group rows), largest first.  A call takes the configuration with the
// best estimated throughput for its tile count (the size-based kernel choice
// of the SGEMM summary's results section, retuned for 256 CUs).
typedef S32Tile<256, 256, 32, 2, 4, 2, 8, true> F32Huge; // 8 waves, 128 KB LDS, 1 WG/CU
typedef S32Tile<256, 128, 32, 4, 2, 3, 8, true> F32Big;  // 8 waves, 144 KB LDS, 1 WG/CU
typedef S32Tile<128, 128, 16, 2, 2, 3, 8, true> F32Mid;  // 4 waves,  48 KB LDS, 3 WG/CU
typedef S32Tile<128, 128, 16, 2, 2, 3, 8> F32MidB;       // the same, loads issued together
typedef S32Tile<64, 64, 32, 1, 1, 3, 8> F32Small;     // 1 wave,   48 KB LDS, 3 WG/CU
typedef S32Tile<64, 64, 32, 2, 2, 3, 8> F32Quad;      // 4 waves of 32x32, 48 KB LDS, 3 WG/CU
typedef S32Tile<128, 64, 32, 2, 2, 3, 8> F32Half;     // 4 waves of 64x32, 72 KB LDS, 2 WG/CU
typedef S32Tile<64, 64, 64, 2, 2, 2, 8> F32QuadK;   // the same in 64-k steps, 64 KB LDS, 2 WG/CU
typedef S32Tile<32, 32, 64, 1, 1, 2, 8> F32TinyK;   // 1 wave, 64-k steps, 32 KB LDS, 5 WG/CU
typedef S32Tile<32, 32, 32, 1, 1, 3, 8> F32Tiny;      // 1 wave,   24 KB LDS, 6 WG/CU

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
  // element pairs (8 bytes) when a leading dimension is even but 16-byte
  // loads are out
  pl.vec_a = va ? 4 : (!c.force_scalar && vec_ok(c.A, c.lda, 2, 4) ? 2 : 1);
  pl.vec_b = vb ? 4 : (!c.force_scalar && vec_ok(c.B, c.ldb, 2, 4) ? 2 : 1);
  pl.vec_c = vc ? T::FN : 1;
  const long long tm = (c.M + T::BM - 1) / T::BM;
  const long long tn = (c.N + T::BN - 1) / T::BN;
  pl.blocks = c.tile_count > 0 ? c.tile_count : tm * tn;
  pl.splits = 1;
  pl.tail = 1;
  pl.ws_bytes = 0;
  return pl;
}

template <class T>
static GemmParams make_params(const Call &c, const Plan &pl) {
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
  p.splits = c.splits;
  p.k_chunk = c.k_chunk;
  p.split_stride = c.split_stride;
  p.vec_ab = vec_bits(pl.vec_a, pl.vec_b, 4);
  p.tile_base = c.tile_base;
  p.tile_count = c.tile_count;
  p.c_tiles = c.c_tiles ? 1 : 0;
  return p;
}

template <class T, bool TA, bool TB, bool VC>
static hipError_t launch_variant(const Call &c, const Plan &pl) {
  const GemmParams p = make_params<T>(c, pl);
  hipLaunchKernelGGL((sgemm_mfma<T, TA, TB, VC>), dim3((unsigned)(pl.blocks * c.splits)),
                     dim3(T::NT), 0, c.stream, p);
  return hipGetLastError();
}

// A Stream-K launch of configuration T over `blocks` workgroups (see
// sgemm_streamk), followed by nothing: the caller runs the fix-up.
template <class T, bool TA, bool TB, bool VC>
static hipError_t launch_streamk_variant(const Call &c, const Plan &pl, const StreamKRun &sk,
                                         long long blocks) {
  const GemmParams p = make_params<T>(c, pl);
  hipLaunchKernelGGL((sgemm_streamk<T, TA, TB, VC>), dim3((unsigned)blocks), dim3(T::NT), 0,
                     c.stream, p, sk);
  return hipGetLastError();
}

template <class T>
static hipError_t dispatch_streamk(const Call &c, const StreamKRun &sk, long long blocks) {
  const Plan pl = make_plan<T>(c, "");
  const int key = (c.ta ? 4 : 0) | (c.tb ? 2 : 0) | (pl.vec_c > 1 ? 1 : 0);
  switch (key) {
    case 0: return launch_streamk_variant<T, false, false, false>(c, pl, sk, blocks);
    case 1: return launch_streamk_variant<T, false, false, true>(c, pl, sk, blocks);
    case 2: return launch_streamk_variant<T, false, true, false>(c, pl, sk, blocks);
    case 3: return launch_streamk_variant<T, false, true, true>(c, pl, sk, blocks);
    case 4: return launch_streamk_variant<T, true, false, false>(c, pl, sk, blocks);
    case 5: return launch_streamk_variant<T, true, false, true>(c, pl, sk, blocks);
    case 6: return launch_streamk_variant<T, true, true, false>(c, pl, sk, blocks);
    default: return launch_streamk_variant<T, true, true, true>(c, pl, sk, blocks);
  }
}

template <class T>
static hipError_t dispatch(const Call &c) {
  const Plan pl = make_plan<T>(c, "");
  if (pl.blocks * c.splits > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int key = (c.ta ? 4 : 0) | (c.tb ? 2 : 0) | (pl.vec_c > 1 ? 1 : 0);
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

template <class T>
static long long tiles_of(const Call &c) {
  return (long long)((c.M + T::BM - 1) / T::BM) * (long long)((c.N + T::BN - 1) / T::BN);
}

enum class F32Cfg { kHuge, kBig, kMid, kMidB, kSmall, kTiny, kQuad, kHalf, kQuadK, kTinyK };

// Share of the machine a configuration keeps busy: with T tiles spread over
// the CUs, the busiest CU holds ceil(T/CUs) of them while the average is
// T/CUs (several workgroups per CU share it, so only whole tiles per CU
// count).
static double busy_share(long long tiles) {
  const double per_cu = (double)tiles / kCUs;
  const double rounds = (double)((tiles + kCUs - 1) / kCUs);
  return per_cu / rounds;
}

// Share of a busy CU's four SIMDs that hold a wave: the workgroups resident
// on it at once (at most `per_cu`, the LDS limit) times the waves of each.
// A multi-wave tile built to share its CU (per_cu > 1) runs below its
// measured efficiency when it is alone there: nothing else hides its load
// waits (the 128x128 tile at 1792^3..2048^3 with one workgroup per CU ran
// 5-7% behind the same tile split twice, two per CU).
template <class T>
static double simd_share(long long tiles, int per_cu) {
  long long resident = (tiles + kCUs - 1) / kCUs;
  if (resident > per_cu) resident = per_cu;
  const double waves = (double)(resident * T::NWAVES);
  if (per_cu > 1 && T::NWAVES >= 4 && resident == 1) return 0.88;
  return waves >= 4.0 ? 1.0 : waves / 4.0;
}

// Throughput score of configuration T when its tiles are run `splits` times
// (one per K chunk): measured throughput at full occupancy x the two shares.
template <class T>
static double score_of(const Call &c, double eff, int per_cu, int splits) {
  const long long t = tiles_of<T>(c) * splits;
  return eff * busy_share(t) * simd_share<T>(t, per_cu);
}

// K chunk of configuration T when K is split `splits` ways: whole K steps.
template <class T>
static int chunk_of(const Call &c, int splits) {
  return ((c.K + splits - 1) / splits + T::BK - 1) / T::BK * T::BK;
}

// The 32x32 tile's throughput depends on the K each workgroup runs: one wave
// per workgroup, so its prologue and epilogue weigh like ~700 k of work
// (measured 0.435 of the peak at K = 1024, 0.41 at 1536, 0.63 at 4096).
static double tiny_eff(int kc) { return 0.74 * (double)kc / ((double)kc + 700.0); }

struct F32Choice {
  F32Cfg cfg;
  int splits;   // wanted K chunks (1 = none); clamp_splits has the last word
  double time;  // estimated seconds
  int tail;     // K chunks of the last round's tiles (1 = the round runs whole)
  int sk = 0;   // Stream-K mode (streamk_geometry; 0 = none)
};

// Estimated time of a choice: the product at `score` of the fp32 peak, plus,
// when K is split S ways, the extra pass: a few microseconds to launch and S
// fp32 slabs of M x N written and read back at ~6 TB/s (the writes overlap the
// product).
static double est_time(const Call &c, double score, int splits) {
  const double flops = 2.0 * (double)c.M * (double)c.N * (double)c.K;
  double t = flops / (score * 157.3e12);
  if (splits > 1) t += 4e-6 + 8.0 * splits * (double)c.M * (double)c.N / 6e12;
  return t;
}

// Best split of K for configuration T, if one is estimated faster than
// `best`: chunks of at least `kmin` (so each workgroup still runs enough K
// steps to hide its prologue and epilogue), at most 8.
// Each workgroup also pays a fixed cost for its prologue and epilogue, about
// k0 = 100 k of work for the 128x128 tile, which its co-resident workgroups
// hide while all of a CU's workgroups fit on it at once and which longer
// chunks amortise.  A split into chunks shorter than 512 k that puts more
// workgroups on a CU than fit (so they run in rounds, each paying it again)
// has its product time scaled by (1 + k0/kc) / (1 + k0/K), its fixed cost
// relative to the same tile unsplit.  Measured (sweep protocol, interleaved):
// 1792^3, 5 chunks of 368 k at 3.8 workgroups per CU, ran at 81.5 TFLOP/s
// against 92 unsplit; applied to longer chunks too, the rule cost 3-10% at
// 2176^3 (544 k), 2304^3, 2560^3 and 3200^3, where the split pays.
template <class T>
static void try_splits(const Call &c, F32Cfg cfg, double eff, int per_cu, int kmin,
                       F32Choice &best, double k0 = 0.0) {
  for (int S = 2; S <= 8; ++S) {
    const int kc = chunk_of<T>(c, S);
    if (kc < kmin) break;
    const int used = (c.K + kc - 1) / kc;
    const double e = cfg == F32Cfg::kTiny ? tiny_eff(kc) : eff;
    const bool rounds = kc < 512 && tiles_of<T>(c) * used > (long long)per_cu * kCUs;
    const double fixed = rounds ? (1.0 + k0 / kc) / (1.0 + k0 / c.K) : 1.0;
    const double t = est_time(c, score_of<T>(c, e, per_cu, used) / fixed, used);
    if (t < best.time * 0.98) best = F32Choice{cfg, used, t, 1};
  }
}

// The last round.  T tiles fill floor(T/CUs) whole rounds (whole tiles per
// CU, the busy share's unit); the r = T mod CUs tiles left over would keep r
// CUs busy for a whole tile's time while the others idle.  Run instead as a
// split-K pass of S chunks of kc k over the CUs, they cost each CU
// ceil(r*S/CUs) workgroups of (kc + k0)/K of a tile's time, k0 being a
// workgroup's prologue and epilogue in k units (measured: ~700 for the large
// tile, which runs alone on its CU, ~200 for the medium one, whose
// co-resident workgroups hide most of it), plus a second launch and the
// reduction of r*S dense fp32 tile blocks.  The medium tile needs two whole
// rounds first (with one tile per CU its rounds run below the measured
// efficiency).  The best split is taken when it beats the choice so far by 1%
// (measured over the 93 sizes of the square sweep, the model's picks gain up
// to 13% and lose nowhere more than run-to-run variation).
template <class T>
static void try_tail(const Call &c, F32Cfg cfg, double eff, int per_cu, int min_rounds, double k0,
                     F32Choice &best) {
  const long long tiles = tiles_of<T>(c);
  const long long full = tiles / kCUs * kCUs;
  const int rest = (int)(tiles - full);
  if (full < (long long)min_rounds * kCUs || rest == 0 || rest * 2 > kCUs) return;
  const double flops = 2.0 * (double)c.M * (double)c.N * (double)c.K;
  const double whole = (double)tiles / kCUs;   // tiles per CU on average
  const double simd = simd_share<T>(full, per_cu);
  F32Choice pick{cfg, 1, 0.0, 1};
  for (int S = 2; S <= 16; ++S) {
    const int kc = chunk_of<T>(c, S);
    if (kc < 128) break;
    const int used = (c.K + kc - 1) / kc;
    const long long wgs = (long long)rest * used;
    const double tail = (double)((wgs + kCUs - 1) / kCUs) * ((double)kc + k0) / (double)c.K;
    const double busy = whole / ((double)(full / kCUs) + tail);
    const double extra = (double)wgs * T::BM * T::BN * 4.0 * 2.0 +
                         (double)rest * T::BM * T::BN * 4.0 * (c.beta != 0.0f ? 2.0 : 1.0);
    const double t = flops / (eff * busy * simd * 157.3e12) + 8e-6 + extra / 6e12;
    if (pick.tail == 1 || t < pick.time) pick = F32Choice{cfg, 1, t, used};
  }
  if (pick.tail > 1 && pick.time < best.time * 0.99) best = pick;
}

// Calls with an operand that cannot take 16-byte loads (leading dimension or
// base not a multiple of 4 floats) run the register-staged, element-wise load
// path, whose workgroups wait on their loads much longer than the direct
// path's, so the estimate above does not hold for them.  Measured on seven
// such shapes (interleaved, every tile and split): the 128x128 tile alone on
// a CU, or two or three sharing it, each cost about 0.106, 0.175 and 0.221
// us per k of work, plus a fixed ~110 k (alone) or ~44 k (shared) for the
// prologue and epilogue; the other tiles ran behind it.  The chosen K split
// S (1..8, chunks of at least 128 k) minimises the busiest CU's time, its
// workgroups taken in groups of three, plus the split's second pass
// (S fp32 slabs written and read, C read and written, at ~5 TB/s).  Against
// the direct-path estimate: 1000x3000x517 +15%, 2000x2000x1000 +15%,
// 3000^3 +10%, 1500^3 +10%, 1000^3 +41%, 517x3000x1000 +89%.  Grids of three
// or more 128x128 tiles per CU keep the direct-path choice: there the large
// tiles, staged, run ahead (4096^3 126 against 110 TFLOP/s, 8000^3 118
// against 111).
// (The element-wise load switch for tests does not count: it changes how the
// data moves, never the tile or the K split, so results stay bitwise equal.)
static bool staged_call(const Call &c) {
  return !vec_ok(c.A, c.lda, 4, 4) || !vec_ok(c.B, c.ldb, 4, 4);
}

static F32Choice choose_staged(const Call &c) {
  static const double us_per_k[4] = {0.0, 0.106e-6, 0.175e-6, 0.221e-6};
  const long long tiles = tiles_of<F32Mid>(c);
  const double mn_bytes = (double)c.M * (double)c.N * 4.0;
  F32Choice best{F32Cfg::kMid, 1, 0.0, 1};
  for (int S = 1; S <= 8; ++S) {
    const int kc = S == 1 ? c.K : chunk_of<F32Mid>(c, S);
    if (S > 1 && kc < 128) break;
    const int used = S == 1 ? 1 : (c.K + kc - 1) / kc;
    const long long n = (tiles * used + kCUs - 1) / kCUs;   // busiest CU's workgroups
    const double k0 = n == 1 ? 110.0 : 44.0;
    double t = ((double)kc + k0) * ((double)(n / 3) * us_per_k[3] + us_per_k[n % 3]);
    t += used > 1 ? 4e-6 + (2.0 * used + 2.0) * mn_bytes / 5e12
                  : (c.beta != 0.0f ? 2.0 : 1.0) * mn_bytes / 5e12;
    if (S == 1 || t < best.time) best = F32Choice{F32Cfg::kMid, used, t, 1};
  }
  if (tiles * best.splits > kCUs) best.cfg = F32Cfg::kMidB;
  return best;
}

// Otherwise score = measured throughput at full occupancy (fraction of the
// fp32 peak at 4096^3, same-process interleaved timing: 0.92, 0.91, 0.57,
// and tiny_eff for the 32x32 tile) x the two shares above; the largest score
// wins.  Last, an unsplit 256x128 choice gives way to the 256x256 tile
// (unsplit, or with its own last-round split) when that is estimated no
// slower at efficiency 0.95: measured over the square sweep (interleaved
// A/B), it runs 2-3.5% ahead wherever it replaces an unsplit 256x128 call
// (4096^3 149.5 vs 144.4, 8192^3 151.2 vs 146.7), but falls 2-8% behind
// where the 256x128 or 128x128 tile has a last-round or whole split that
// evens out its rounds, so it is offered only in place of the former.  When K is at least max(M, N) and 1024, K splits of every
// configuration are estimated too (est_time; measured
// winners: 1536^3, 2560^3, 3072^3 and deep-K shapes such as 1024 x 1024 x
// 8192 take 3-8 chunks of the 128x128 tile; square problems up to 1024 and
// those whose tiles already fill the CUs stay unsplit).
// Stream-K mode (streamk_geometry) for a call that takes the four-wave 64x64
// tile whole (0: the plain launch).  By size: past two whole rounds of one
// tile per CU, with r leftover tiles, at most half the CUs, the whole rounds
// run as whole tiles and the leftover tiles' K steps are dealt out to one
// more workgroup per CU (mode 5).  The plain launch gives r CUs one tile
// more than the others; the leftover's K steps spread over every CU
// instead, and the Stream-K workgroups run beside the whole tiles (three of
// these workgroups fit on a CU).  Measured, plain -> Stream-K, TFLOP/s, beta
// 1, interleaved; first back to back, then with a 512 MiB cache flush before
// each call: 1472^3 85.4 -> 95.0 and 80.9 -> 88.9, 1536^3 93.6 -> 103.6 and
// 88.8 -> 96.6, 1600^3 101.7 -> 106.3 and 96.1 -> 98.4, 2048x1152x1024
// 88.4 -> 91.4 and 82.2 -> 83.9, 1152x2048x1536 93.4 -> 103.9.  Past one
// round only it gained back to back (1088^3 58.3 -> 61.6, 1152^3 67.9 ->
// 70.3) but not after a flush (57.3 -> 56.2, 63.4 -> 63.1), so those stay
// plain; with larger leftovers it lost (1664^3 and 1216^3 +-1%, 1280^3 -2%,
// 1408^3 -8%, 1728^3 -5%), and so did dealing out every tile's K steps with
// no whole tiles first (1408^3 -15%, 1664^3 -8%, 1536^3 +4%: most tiles
// were then shared, and their partial sums went through memory).
static int streamk_of(const Call &c) {
  if (c.streamk_mode >= 2) return c.streamk_mode;
  if (c.streamk_mode == 1) return 0;
  const long long tiles = tiles_of<F32Quad>(c);
  if (tiles <= 2LL * kCUs || tiles > 3LL * kCUs) return 0;
  const long long r = tiles % kCUs;
  return r > 0 && 2 * r <= kCUs ? 5 : 0;
}

// Stream-K behind whole rounds (mode 5) in place of the model's choice
// `best`, for calls with 1024 <= K <= 2 max(M, N) and rows that take 16-byte
// loads (deeper K keeps the model's K splits, which were not measured
// against it).  The r leftover tiles' K steps go to one more workgroup per
// CU in the same launch, so every CU ends with the same work.  Measured
// (interleaved, a 512 MiB flush before each call, beta 1, TFLOP/s, on two
// boxes, one of which held its package power limit most of the time):
// - the 128x128 tile with Stream-K, whatever was chosen, for 2 to 7 rounds
//   of its tiles and r from a quarter to seven eighths of the CUs: 3328^3
//   (256x128 tile split 3) 127.0 -> 135.4, 3840^3 (256x256 tile) 128.1 ->
//   139.4, 4352^3 (128x128 tile) 131.0 -> 141.7, 4864^3 (256x128 tile) 134.7
//   -> 142.1, 5248^3 136.5 -> 144.5 (a K split there too: 3200^3 131.1 ->
//   132.7); both boxes gained.  Past about seven
//   rounds the runs are long enough for the power-limited box to clock the
//   128x128 tile ~5% below the larger tiles (2.20-2.25 against 2.33-2.38
//   GHz), so
// - from 7 to 16 rounds it replaces only the 128x128 tile itself (plain or
//   with the last round split): 6016^3 139.4 -> 145.0, 7040^3 142.4 ->
//   145.3, 7296^3 141.2 -> 144.7; with a leftover of a few tiles the last
//   round's split did as well or better (2944^3 128.6 against 126.8,
//   4608^3 141.8 against 139.5), with a nearly full last round the plain
//   launch is balanced already (4992^3 -0.8%, 5760^3 -0.3%), and past 16
//   rounds the imbalance is small (9344^3 145.0 against 144.5);
// - the 256x128 and 256x256 tiles, plain or with the last round split, take
//   Stream-K on the same tile whenever a round is left partly filled: over
//   35 sweep sizes from 3328^3 to 12672^3 none lost more than 0.2%, 4864^3
//   134.7 -> 139.7, 5632^3 139.8 -> 144.5, 6400^3 140.5 -> 142.1, 10752^3
//   146.2 -> 147.6, the last-round splits' sizes +0.2% on average;
// - ahead of all of these, the 256x256 tile (Stream-K when a round is left
//   partly filled) wherever it has at least one round of tiles and at least
//   97% of its tiles' area lies inside the matrix: in place of the 128x128
//   tile, 6144^3 147.2 -> 148.9, 8448^3 144.6 -> 149.8, 9472^3 144.1 ->
//   150.4, 11008^3 145.1 -> 151.2, 12800^3 145.7 -> 150.5 (n a multiple of
//   256: no tile area lost), 9344^3 142.5 -> 146.2, 12416^3 144.2 -> 148.3
//   (half-empty last tiles, 97-98% of the area inside); at 96-96.5%
//   (6528^3 .. 7296^3) it lost 0.3-1.6% and is not taken.  Both boxes hold
//   this tile's clock highest.  The model's efficiencies, measured at
//   4096^3 in short runs, count neither the area of half-empty edge tiles
//   nor the lower clock of the smaller tiles over long runs.
template <class T>
static bool streamk_fits(const Call &c, int mode, StreamKRun &sk, long long &blocks);

// The choice with Stream-K mode 5 on configuration T, if its partial blocks
// fit the call's workspace; else `best` (which may split the last round in
// less workspace).
template <class T>
static F32Choice streamk_if_fits(const Call &c, F32Cfg cfg, const F32Choice &best) {
  StreamKRun sk;
  long long blocks = 0;
  return streamk_fits<T>(c, 5, sk, blocks) ? F32Choice{cfg, 1, best.time, 1, 5} : best;
}

static F32Choice streamk_instead(const Call &c, const F32Choice &best) {
  const long long mx = c.M > c.N ? c.M : c.N;
  if (c.split_mode != 0 || c.tail_mode != 0 || c.streamk_mode != 0 || c.K < 1024 ||
      (long long)c.K > 2 * mx || staged_call(c))
    return best;
  // The 256x256 tile, with Stream-K when its last round is partly filled,
  // wherever it has a round of tiles and at least 97% of its tiles' area
  // lies inside the matrix.
  const long long th = tiles_of<F32Huge>(c);
  const double useful = (double)c.M * (double)c.N / ((double)th * F32Huge::BM * F32Huge::BN);
  if (th >= kCUs && useful >= 0.97) {
    if (th % kCUs == 0) return F32Choice{F32Cfg::kHuge, 1, best.time, 1, 0};
    return streamk_if_fits<F32Huge>(c, F32Cfg::kHuge, best);
  }
  const long long tm = tiles_of<F32MidB>(c);
  const long long r = tm % kCUs;
  const bool whole_k = best.splits == 1;   // unsplit, or only the last round split
  const bool mid = whole_k && (best.cfg == F32Cfg::kMid || best.cfg == F32Cfg::kMidB);
  if (tm >= 2LL * kCUs && 4 * r >= kCUs && 8 * r <= 7LL * kCUs &&
      (tm <= 7LL * kCUs || (mid && tm <= 16LL * kCUs)))
    return streamk_if_fits<F32MidB>(c, F32Cfg::kMidB, best);
  if (!whole_k) return best;
  if (best.cfg == F32Cfg::kHuge && tiles_of<F32Huge>(c) >= kCUs && tiles_of<F32Huge>(c) % kCUs != 0)
    return streamk_if_fits<F32Huge>(c, F32Cfg::kHuge, best);
  if (best.cfg == F32Cfg::kBig && tiles_of<F32Big>(c) >= kCUs && tiles_of<F32Big>(c) % kCUs != 0)
    return streamk_if_fits<F32Big>(c, F32Cfg::kBig, best);
  return best;
}

static F32Choice choose_f32(const Call &c) {
  const int forced = c.split_mode >= 2 ? c.split_mode : 1;
  const int tail = c.tail_mode >= 2 && forced == 1 ? c.tail_mode : 1;
  const int fsk = forced == 1 && tail == 1 && c.streamk_mode >= 2 ? c.streamk_mode : 0;
  if (c.tile_config == 1) return F32Choice{F32Cfg::kBig, forced, 0.0, tail, fsk};
  if (c.tile_config == 2) return F32Choice{F32Cfg::kMid, forced, 0.0, tail};
  if (c.tile_config == 3) return F32Choice{F32Cfg::kSmall, forced, 0.0, tail};
  if (c.tile_config == 4) return F32Choice{F32Cfg::kTiny, forced, 0.0, tail};
  if (c.tile_config == 5) return F32Choice{F32Cfg::kMidB, forced, 0.0, tail, fsk};
  if (c.tile_config == 6) return F32Choice{F32Cfg::kHuge, forced, 0.0, tail, fsk};
  if (c.tile_config == 7)
    return F32Choice{F32Cfg::kQuad, forced, 0.0, tail, forced == 1 && tail == 1 ? streamk_of(c) : 0};
  if (c.tile_config == 8) return F32Choice{F32Cfg::kHalf, forced, 0.0, tail, fsk};
  if (c.tile_config == 9) return F32Choice{F32Cfg::kQuadK, forced, 0.0, tail};
  if (c.tile_config == 10) return F32Choice{F32Cfg::kTinyK, forced, 0.0, tail};
  if (c.split_mode == 0 && c.tail_mode == 0 && staged_call(c) && tiles_of<F32Tiny>(c) > kCUs &&
      tiles_of<F32Mid>(c) < 3LL * kCUs)
    return choose_staged(c);
  // Grids of one to three 64x64 tiles per CU (all resident at once) whose K
  // is not deep: the 64x64 tile of four 32x32 waves, unsplit.  Each CU then
  // holds four to twelve waves with no split pass, where the 128x128 tile
  // needs a K split (and its reduction) to fill the CUs and the 32x32 tile
  // runs a single wave per workgroup.  Measured (interleaved, beta 1 and 0)
  // against the choice before it: 1024^3 56 -> 78 TFLOP/s, 1280^3 80 -> 85,
  // 1408^3 88 -> 103, 1536^3 90 -> 93, 1664^3 105 -> 110,
  // 2048x1024x1024 83 -> 103, 1536x1024x1024 65 -> 78, 2048x512x2048
  // 79-84 -> 86, 1000^3 and 4096x256x1024 +1-3%; 1152^3 71 -> 68 is the one
  // loss.  Deeper K (1024x1024x4096) keeps the 128x128 tile in 8 chunks
  // (106 against 93), and 1792^3 (3.1 tiles per CU) the unsplit 128x128 tile.
  // Past three of those per CU, grids of 1.5 to 2 128x64 tiles per CU (both
  // resident at once) take that tile, four 64x32 waves, unsplit: measured
  // against the 128x128 tile chosen before (beta 1 and 0), 1792^3 90-97 ->
  // 99-100 TFLOP/s, 1920^3 110 -> 114-116, 2048^3 124-125 -> 130-131,
  // 1800x1900x2000 95-97 -> 101-104, 1024x4096x1024 116-119 -> 120-124,
  // 4096x1024x2048 +3-4%, 2048x2048x512 +5%, 2560x1280x1280 +2%.
  // Up to two 64x64 tiles per CU the tile runs in 64-k steps through two LDS
  // slots (64 KB, so two of its workgroups share a CU): half the steps, and
  // half the barriers, per tile.  Measured (interleaved, a 512 MiB flush
  // before each call, beta 1, TFLOP/s, 32-k steps in three slots -> this):
  // 1024^3 68.0 -> 73.9, 1000^3 59.9 -> 64.0, 1024x1024x2048 80.2 -> 89.3,
  // 1152^3 63.9 -> 65.8, 1280^3 80.2 -> 82.1, 1408^3 97.5 -> 100.7, 896^3
  // 51.0 -> 55.3; past two per CU the third workgroup no longer fits and
  // three 32-k slots stay ahead (1664^3 104.9 against 98.8), as did 64-k
  // steps in three slots (one workgroup per CU: 1024^3 71.5, 1408^3 81.7).
  if (c.split_mode == 0 && c.tail_mode == 0 && !staged_call(c)) {
    const long long q = tiles_of<F32Quad>(c), h = tiles_of<F32Half>(c);
    const long long mx = c.M > c.N ? c.M : c.N;
    if ((long long)c.K <= 2 * mx) {
      if (q >= kCUs && q <= 3LL * kCUs) {
        const int sk = streamk_of(c);
        return F32Choice{sk == 0 && q <= 2LL * kCUs ? F32Cfg::kQuadK : F32Cfg::kQuad, 1, 0.0, 1, sk};
      }
      // Three whole rounds and at most a third of a round more: the same tile
      // with Stream-K behind the whole rounds (the leftover's K steps over one
      // more workgroup per CU), in place of the 128x64 tile.  Measured
      // (interleaved, flush before each call, TFLOP/s, 128x64 -> this):
      // 1760^3 (784 tiles) 88.7 -> 100.0, 1792^3 94.7 -> 105.1, 2048 x 1600 x
      // 1800 (800) 93.7 -> 103.9, 1700x1900x1500 (810) 89.2 -> 96.5, 1856^3
      // (841) 99.5 -> 104.7, 1792x1920x1792 (840) 100.7 -> 104.5; from half a
      // round more it lost (1920^3, 900 tiles, 108.6 against 101.6; 1984^3
      // 114.1 against 98.4).
      StreamKRun skr;
      long long skb = 0;
      const int sk3 = c.streamk_mode >= 2 ? c.streamk_mode : 5;
      if (q > 3LL * kCUs && 3 * (q - 3LL * kCUs) <= kCUs && c.streamk_mode != 1 &&
          streamk_fits<F32Quad>(c, sk3, skr, skb))
        return F32Choice{F32Cfg::kQuad, 1, 0.0, 1, sk3};
      if (2 * h >= 3LL * kCUs && h <= 2LL * kCUs) return F32Choice{F32Cfg::kHalf, 1, 0.0, 1};
      // Exactly two full rounds of the 64x64 tile at three resident
      // workgroups per CU (six tiles on every CU), 1024 <= K <= max(M, N):
      // that tile, plain, where the larger tiles leave a round partly filled.
      // Measured (interleaved, flush before each call, beta 1, TFLOP/s, the
      // 256x128 tile chosen before -> this): 1536x4096x1536 99.0 -> 124.0,
      // 1024x6144x1024 94.4 -> 116.6, 4096x1536x2048 102.1 -> 127.6 (the
      // 128x64 tile ran 120.0, 112.5, 123.6 there).
      if (q == 6LL * kCUs && c.K >= 1024 && c.K <= mx)
        return F32Choice{F32Cfg::kQuad, 1, 0.0, 1};
      // Two to three and a half rounds of 128x64 tiles, a round partly
      // filled, both sides and K at least 640: that tile with Stream-K
      // behind the whole rounds, in place of any other choice.  Measured
      // (interleaved, flush before each call, beta 1, TFLOP/s, the choice
      // before -> this): 2176^3 (578 tiles; 128x128 split 4) 104.9 -> 119.1,
      // 2304^3 (648; split 3) 114.0 -> 119.8, 2432^3 (722) 118.1 -> 119.7,
      // 2560^3 (800) 116.7 -> 121.6, 2688^3 (882; 256x128) 119.3 -> 125.9,
      // 2048x2304x2048 (576; 32x32) 93.6 -> 120.6, 2560x2048x2560 118.6 ->
      // 123.1, 2176x2176x1536 (256x128) 75.4 -> 112.3, 1536x3072x2048
      // (32x32) 93.7 -> 120.8; narrow and short calls as well: 768 x 6144 x
      // 2048 (32x32) 93.2 -> 120.3, 640x8192x1536 (256x128) 82.9 -> 113.7,
      // 896x5120x3000 91.4 -> 121.3, 2176x2176x768 68.5 -> 90.6,
      // 3072x1536x640 65.2 -> 86.0.  At K = 512 it lost (2560x2560x512 84.6
      // against 79.7).  The tile alone, without Stream-K, lost at most of
      // these (2176^3 94.7, 2560^3 103.8).
      const long long mn = c.M < c.N ? c.M : c.N;
      if (h > 2LL * kCUs && 2 * h <= 7LL * kCUs && h % kCUs != 0 && c.K >= 640 && mn >= 640 &&
          c.streamk_mode != 1 && streamk_fits<F32Half>(c, sk3, skr, skb))
        return F32Choice{F32Cfg::kHalf, 1, 0.0, 1, sk3};
    }
  }
  const double big = score_of<F32Big>(c, 0.92, 1, 1);
  const double mid = score_of<F32Mid>(c, 0.91, 3, 1);
  const double small = score_of<F32Small>(c, 0.57, 3, 1);
  const double tiny = score_of<F32Tiny>(c, tiny_eff(c.K), 6, 1);
  F32Choice best;
  if (tiles_of<F32Tiny>(c) <= kCUs) {
    // Problems too small to give every CU even a 32x32 tile are
    // latency-bound: the most workgroups and the shortest prologue win.
    best = F32Choice{F32Cfg::kTiny, 1, est_time(c, tiny, 1), 1};
  } else if (big >= mid && big >= small && big >= tiny) {
    best = F32Choice{F32Cfg::kBig, 1, est_time(c, big, 1), 1};
  } else if (mid >= small && mid >= tiny) {
    best = F32Choice{F32Cfg::kMid, 1, est_time(c, mid, 1), 1};
  } else {
    best = small >= tiny ? F32Choice{F32Cfg::kSmall, 1, est_time(c, small, 1), 1}
                         : F32Choice{F32Cfg::kTiny, 1, est_time(c, tiny, 1), 1};
  }
  if (c.split_mode == 0 && c.K >= 1024 && c.K >= (c.M > c.N ? c.M : c.N)) {
    // The large tile runs one workgroup per CU, so nothing overlaps its
    // prologue and epilogue: it needs longer chunks than the others.
    try_splits<F32Big>(c, F32Cfg::kBig, 0.92, 1, 1024, best);
    try_splits<F32Mid>(c, F32Cfg::kMid, 0.91, 3, 256, best, 100.0);
    try_splits<F32Small>(c, F32Cfg::kSmall, 0.57, 3, 1024, best);
    try_splits<F32Tiny>(c, F32Cfg::kTiny, 0.63, 6, 1024, best);
  } else if (c.split_mode == 0 && c.K >= 512 && c.K < (c.M > c.N ? c.M : c.N) &&
             tiles_of<F32Mid>(c) < kCUs) {
    // Wide, short problems whose 128x128 tiles leave CUs idle: that tile in
    // chunks of at least 512 k beats the small tiles' many workgroups
    // (interleaved: 517x3000x1000 +13%, 256x4096x2048 +7%, 256x8192x1024
    // +33%, 128x16384x4096 +65%); with shorter chunks it fell behind
    // (384x3000x600 in chunks of 304: -21%).
    try_splits<F32Mid>(c, F32Cfg::kMid, 0.91, 3, 512, best);
  } else if (c.split_mode >= 2) {
    best.splits = forced;
  }
  if (c.split_mode == 0 && c.tail_mode == 0) {
    try_tail<F32Big>(c, F32Cfg::kBig, 0.92, 1, 1, 700.0, best);
    try_tail<F32Mid>(c, F32Cfg::kMid, 0.91, 3, 2, 200.0, best);
  } else if (c.tail_mode >= 2 && best.splits == 1) {
    best.tail = c.tail_mode;
  }
  if (c.split_mode == 0 && c.tail_mode == 0 && best.cfg == F32Cfg::kBig && best.splits == 1 &&
      best.tail == 1) {
    F32Choice h{F32Cfg::kHuge, 1, est_time(c, score_of<F32Huge>(c, 0.95, 1, 1), 1), 1};
    try_tail<F32Huge>(c, F32Cfg::kHuge, 0.95, 1, 1, 700.0, h);
    if (h.time <= best.time) best = h;
  }
  // Spread loads pay while a CU holds one workgroup; with several resident
  // the others hide the load bursts and issuing them together is cheaper.
  if (best.cfg == F32Cfg::kMid && tiles_of<F32Mid>(c) * best.splits > kCUs) best.cfg = F32Cfg::kMidB;
  // Grids of 170 to 255 64x64 tiles (two thirds of a round to just under
  // one) with K <= 1.5 max(M, N): the 64x64 tile of four 32x32 waves,
  // unsplit, in place of the 32x32 tile when that tile would put a fourth
  // workgroup on some CUs, and in place of a K split when K <= 1536.
  // Measured (interleaved, a 512 MiB flush before each call, beta 1,
  // TFLOP/s, the choice before -> this): 896^3 (the 32x32 tile, 784 of
  // them) 39.9 -> 51.0, 928^3 42.9 -> 52.4, 960^3 46.2 -> 59.1, 600 x 1600 x
  // 800 45.0 -> 56.9, 800x1200x1000 44.8 -> 57.9, 1024x768x1024 (the 128x128
  // tile split 4) 41.4 -> 51.6, 1000x700x1200 (split 4) 38.4 -> 45.4, 960 x
  // 1024 x 1400 (split 4) 55.6 -> 67.6, 1500x500x1500 (split 5) 49.9 ->
  // 51.7.  With at most three 32x32 tiles per CU that tile stays ahead
  // (864^3 48.8 against 44.7, 832^3 45.2 against 43.2), and so does the K
  // split for longer K (2048x384x2048 67.9 against 60.4, 768x1024x2048 67.4
  // against 60.8, 896x896x3000 81.4 against 65.2).
  // Under one round of 64x64 tiles, the same tile (64-k steps) also replaces
  // an unsplit larger tile that leaves over half the CUs idle, with K <=
  // max(M, N).  Measured (interleaved, flush before each call, TFLOP/s, the
  // choice before -> this): 512x1024x256 (the 128x128 tile, 32 of them)
  // 10.8 -> 20.1, 200x3000x300 9.5 -> 21.2, 64x8192x512 (the 256x128 tile,
  // 64 of them) 7.6 -> 28.4.  In place of the 32x32 tile at up to three of
  // those per CU it won and lost by a few percent (512^3 16.2 -> 17.3, 768^3
  // 39.2 -> 43.2, but 320^3 5.2 -> 4.8, 448^3 11.6 -> 11.1, 800^3 41.6 ->
  // 38.3), so that tile stays there; deep-K splits stay too (512x512x2048
  // 29.2 against 23.4).
  // The 32x32 tile in 64-k steps through two slots (32 KB, five workgroups
  // per CU) where the model takes that tile with at most 2.25 of them per
  // CU: half the steps, so half the waits and load-issue points.  Measured
  // (interleaved, flush before each call, TFLOP/s, 32-k steps -> this):
  // 512^3 15.8 -> 17.1, 640^3 25.7 -> 27.7, 768^3 37.8 -> 40.5, 384^3 8.1
  // -> 8.6, 256^3 3.0 -> 3.1, 1000x200x1000 13.1 -> 13.9, 256x2048x512 30.2
  // -> 32.2, 300x700x900 13.2 -> 13.7; with more tiles per CU the 32-k form
  // stayed ahead (800^3 41.4 against 40.4, 864^3 48.5 against 47.8,
  // 100x5000x400 21.4 against 20.6).
  if (c.split_mode == 0 && c.tail_mode == 0 && !staged_call(c) && best.cfg == F32Cfg::kTiny &&
      best.splits == 1 && best.tail == 1 && 4 * tiles_of<F32Tiny>(c) <= 9LL * kCUs)
    best.cfg = F32Cfg::kTinyK;
  if (c.split_mode == 0 && c.tail_mode == 0 && !staged_call(c)) {
    const long long q = tiles_of<F32Quad>(c);
    const long long mx = c.M > c.N ? c.M : c.N;
    if (q >= 170 && q < kCUs && 2LL * c.K <= 3 * mx &&
        ((best.cfg == F32Cfg::kTiny && tiles_of<F32Tiny>(c) > 3LL * kCUs) ||
         (best.splits > 1 && c.K <= 1536)))
      return F32Choice{F32Cfg::kQuadK, 1, best.time, 1};
    if (q < kCUs && best.splits == 1 && best.tail == 1) {
      long long tb = 0;
      if (best.cfg == F32Cfg::kMid || best.cfg == F32Cfg::kMidB) tb = tiles_of<F32Mid>(c);
      else if (best.cfg == F32Cfg::kBig) tb = tiles_of<F32Big>(c);
      else if (best.cfg == F32Cfg::kHuge) tb = tiles_of<F32Huge>(c);
      if (tb > 0 && 2 * tb < kCUs && q > tb && (long long)c.K <= mx)
        return F32Choice{F32Cfg::kQuadK, 1, best.time, 1};
    }
  }
  return streamk_instead(c, best);
}

// Run configuration T, splitting K when the split count says so: the tiles
// of every K chunk write raw fp32 sums to a pooled workspace, then one pass
// sums the chunks in order and applies alpha and beta.  If the workspace
// cannot be had the call runs unsplit.
// The last round's tiles as a split-K pass (try_tail): the whole rounds run
// as usual, then the r leftover tiles' K chunks write dense fp32 tile blocks
// to a pooled workspace and a reduction combines them into C.  Returns false
// (nothing launched) when the split does not apply or the workspace cannot
// be had; the caller then runs the call whole.
template <class T>
static bool launch_tail(const Call &c, int want, hipError_t *err) {
  const long long tiles = tiles_of<T>(c);
  const long long full = tiles / kCUs * kCUs;
  const int rest = (int)(tiles - full);
  if (want < 2 || full == 0 || rest == 0 || tiles > 0x7fffffffLL) return false;
  Call tc = c;
  tc.tile_base = (int)full;
  tc.tile_count = rest;
  int kc = 0;
  const size_t block = (size_t)T::BM * T::BN;
  const int S = clamp_splits(tc, want, T::BK, rest, &kc, (long long)rest * (long long)block);
  if (S <= 1) return false;
  void *ws = nullptr;
  if (workspace_alloc(c, tail_ws_bytes(S, rest, T::BM, T::BN), &ws) != hipSuccess) return false;
  Call dc = c;
  dc.tile_base = 0;
  dc.tile_count = (int)full;
  hipError_t e = dispatch<T>(dc);
  if (e == hipSuccess) {
    tc.C = ws;
    tc.ldc = T::BN;
    tc.alpha = 1.0f;
    tc.beta = 0.0f;
    tc.splits = S;
    tc.k_chunk = kc;
    tc.split_stride = 0;
    tc.c_tiles = true;
    e = dispatch<T>(tc);
  }
  if (e == hipSuccess) {
    TileReduce r;
    r.W = static_cast<const float *>(ws);
    r.S = S;
    r.tiles = rest;
    r.tile_base = (int)full;
    r.BM = T::BM;
    r.BN = T::BN;
    r.tiles_m = (c.M + T::BM - 1) / T::BM;
    r.tiles_n = (c.N + T::BN - 1) / T::BN;
    r.group_m = T::GROUP_M;
    r.M = c.M;
    r.N = c.N;
    r.alpha = c.alpha;
    r.beta = c.beta;
    r.C = static_cast<float *>(c.C);
    r.ldc = c.ldc;
    r.force_scalar = c.force_scalar;
    e = launch_tile_reduce(r, c.stream);
  }
  const hipError_t f = workspace_free(c, ws);
  *err = e != hipSuccess ? e : f;
  return true;
}

// Stream-K geometry of configuration T.  mode 2..4: every tile's K steps
// dealt out to (mode - 1) workgroups per CU; mode 5, 6: the whole rounds of
// one tile per CU as whole tiles, the leftover tiles' K steps dealt out to
// (mode - 4) more workgroups per CU.  Every Stream-K workgroup runs `iters`
// consecutive K steps of its tiles' combined sequence (the last one fewer),
// at most one tile's steps (more workgroups than asked for when the share
// would be longer); `blocks` workgroups in all.  False when nothing is left to deal out or the
// grid would not fit the kernel's int arithmetic.
template <class T>
static bool streamk_geometry(const Call &c, int mode, StreamKRun &sk, long long &blocks) {
  const long long tiles = tiles_of<T>(c);
  const long long steps = (c.K + T::BK - 1) / T::BK;
  if (tiles < 1 || tiles > 0x7fffffffLL || steps < 1 || tiles * steps > (1LL << 40)) return false;
  const bool hybrid = mode >= 5;
  const long long dp = hybrid ? tiles / kCUs * kCUs : 0;
  const long long total = (tiles - dp) * steps;
  if (total < 1) return false;
  const long long want = (long long)(hybrid ? mode - 4 : mode - 1) * kCUs;
  sk.tiles = (int)tiles;
  sk.steps = (int)steps;
  sk.dp = (int)dp;
  sk.iters = (total + want - 1) / want;
  if (sk.iters > steps) sk.iters = steps;   // a run touches at most two tiles
  sk.W = nullptr;
  blocks = dp + (total + sk.iters - 1) / sk.iters;
  return blocks <= 0x7fffffffLL;
}

// Two fp32 tile blocks per Stream-K workgroup.
static size_t streamk_ws_bytes(const StreamKRun &sk, long long blocks, int bm, int bn) {
  return (size_t)(blocks - sk.dp) * 2 * (size_t)bm * (size_t)bn * sizeof(float);
}

// streamk_geometry, also false when the call's workspace cannot hold the
// partial blocks (the call then runs the plain launch).
template <class T>
static bool streamk_fits(const Call &c, int mode, StreamKRun &sk, long long &blocks) {
  return streamk_geometry<T>(c, mode, sk, blocks) &&
         (long long)streamk_ws_bytes(sk, blocks, T::BM, T::BN) <= ws_available(c);
}

// Run configuration T as Stream-K (sgemm_streamk, then launch_streamk_fixup
// for the tiles several workgroups share).  Returns false (nothing launched)
// when the geometry does not apply or the workspace cannot be had.
template <class T>
static bool launch_streamk(const Call &c, int mode, hipError_t *err) {
  StreamKRun sk;
  long long blocks = 0;
  if (!streamk_fits<T>(c, mode, sk, blocks)) return false;
  void *ws = nullptr;
  if (workspace_alloc(c, streamk_ws_bytes(sk, blocks, T::BM, T::BN), &ws) != hipSuccess) return false;
  sk.W = static_cast<float *>(ws);
  hipError_t e = dispatch_streamk<T>(c, sk, blocks);
  if (e == hipSuccess) {
    StreamKFixup f;
    f.W = sk.W;
    f.tiles = sk.tiles;
    f.tile_base = sk.dp;
    f.steps = sk.steps;
    f.iters = sk.iters;
    f.BM = T::BM;
    f.BN = T::BN;
    f.tiles_m = (c.M + T::BM - 1) / T::BM;
    f.tiles_n = (c.N + T::BN - 1) / T::BN;
    f.group_m = T::GROUP_M;
    f.M = c.M;
    f.N = c.N;
    f.alpha = c.alpha;
    f.beta = c.beta;
    f.C = static_cast<float *>(c.C);
    f.ldc = c.ldc;
    f.force_scalar = c.force_scalar;
    e = launch_streamk_fixup(f, c.stream);
  }
  const hipError_t fe = workspace_free(c, ws);
  *err = e != hipSuccess ? e : fe;
  return true;
}

template <class T>
static hipError_t launch_cfg(const Call &c, int want, int tail = 1) {
  hipError_t te;
  if (tail >= 2 && launch_tail<T>(c, tail, &te)) return te;
  int kc = 0;
  const int S = clamp_splits(c, want, T::BK, tiles_of<T>(c), &kc);
  if (S <= 1) return dispatch<T>(c);
  const int ldw = (c.N + 3) / 4 * 4;
  const long long stride = (long long)c.M * ldw;
  void *ws = nullptr;
  if (workspace_alloc(c, split_ws_bytes(S, c.M, c.N), &ws) != hipSuccess) return dispatch<T>(c);
  Call pc = c;
  pc.C = ws;
  pc.ldc = ldw;
  pc.alpha = 1.0f;
  pc.beta = 0.0f;
  pc.splits = S;
  pc.k_chunk = kc;
  pc.split_stride = stride;
  hipError_t e = dispatch<T>(pc);
  if (e == hipSuccess) {
    SplitReduce r;
    r.W = static_cast<const float *>(ws);
    r.stride = stride;
    r.ldw = ldw;
    r.S = S;
    r.M = c.M;
    r.N = c.N;
    r.alpha = c.alpha;
    r.beta = c.beta;
    r.C = c.C;
    r.ldc = c.ldc;
    r.half_out = false;
    r.force_scalar = c.force_scalar;
    e = launch_splitk_reduce(r, c.stream);
  }
  const hipError_t f = workspace_free(c, ws);
  return e != hipSuccess ? e : f;
}

template <class T>
static Plan plan_cfg(const Call &c, const char *name, int want, int tail) {
  Plan pl = make_plan<T>(c, name);
  int kc = 0;
  pl.tail = 1;
  if (tail >= 2) {
    const long long tiles = tiles_of<T>(c), full = tiles / kCUs * kCUs;
    const int rest = (int)(tiles - full);
    Call tc = c;
    tc.tile_base = (int)full;
    tc.tile_count = rest;
    if (full > 0 && rest > 0)
      pl.tail = clamp_splits(tc, tail, T::BK, rest, &kc,
                             (long long)rest * (long long)(T::BM * T::BN));
    if (pl.tail > 1) {
      pl.splits = 1;
      pl.ws_bytes = tail_ws_bytes(pl.tail, rest, T::BM, T::BN);
      return pl;
    }
  }
  pl.splits = clamp_splits(c, want, T::BK, pl.blocks, &kc);
  pl.ws_bytes = pl.splits > 1 ? split_ws_bytes(pl.splits, c.M, c.N) : 0;
  return pl;
}

// Plan of a Stream-K call of configuration T (false: it does not apply).
template <class T>
static bool plan_streamk(const Call &c, const char *name, int mode, Plan &pl) {
  StreamKRun sk;
  long long blocks = 0;
  if (!streamk_fits<T>(c, mode, sk, blocks)) return false;
  pl = make_plan<T>(c, name);
  pl.streamk = true;
  pl.sk_whole = sk.dp;
  pl.blocks = blocks;
  pl.ws_bytes = streamk_ws_bytes(sk, blocks, T::BM, T::BN);
  return true;
}

static const char *f32_name(F32Cfg cfg) {
  switch (cfg) {
    case F32Cfg::kHuge: return "f32 mfma32x32x2 tile 256x256x32 8 waves 2 slots spread loads";
    case F32Cfg::kBig: return "f32 mfma32x32x2 tile 256x128x32 8 waves 3 slots spread loads";
    case F32Cfg::kMid: return "f32 mfma32x32x2 tile 128x128x16 4 waves 3 slots spread loads";
    case F32Cfg::kMidB: return "f32 mfma32x32x2 tile 128x128x16 4 waves 3 slots";
    case F32Cfg::kSmall: return "f32 mfma32x32x2 tile 64x64x32 1 wave 3 slots";
    case F32Cfg::kQuad: return "f32 mfma32x32x2 tile 64x64x32 4 waves 3 slots";
    case F32Cfg::kHalf: return "f32 mfma32x32x2 tile 128x64x32 4 waves 3 slots";
    case F32Cfg::kQuadK: return "f32 mfma32x32x2 tile 64x64x64 4 waves 2 slots";
    case F32Cfg::kTinyK: return "f32 mfma32x32x2 tile 32x32x64 1 wave 2 slots";
    default: return "f32 mfma32x32x2 tile 32x32x32 1 wave 3 slots";
  }
}

static Plan plan_f32_as_is(const Call &c) {
  const F32Choice ch = choose_f32(c);
  const char *name = f32_name(ch.cfg);
  Plan pl;
  if (ch.sk > 0) {
    switch (ch.cfg) {
      case F32Cfg::kHuge: if (plan_streamk<F32Huge>(c, name, ch.sk, pl)) return pl; break;
      case F32Cfg::kBig: if (plan_streamk<F32Big>(c, name, ch.sk, pl)) return pl; break;
      case F32Cfg::kMidB: if (plan_streamk<F32MidB>(c, name, ch.sk, pl)) return pl; break;
      case F32Cfg::kQuad: if (plan_streamk<F32Quad>(c, name, ch.sk, pl)) return pl; break;
      case F32Cfg::kHalf: if (plan_streamk<F32Half>(c, name, ch.sk, pl)) return pl; break;
      default: break;
    }
  }
  switch (ch.cfg) {
    case F32Cfg::kHuge: return plan_cfg<F32Huge>(c, name, ch.splits, ch.tail);
    case F32Cfg::kBig: return plan_cfg<F32Big>(c, name, ch.splits, ch.tail);
    case F32Cfg::kMid: return plan_cfg<F32Mid>(c, name, ch.splits, ch.tail);
    case F32Cfg::kMidB: return plan_cfg<F32MidB>(c, name, ch.splits, ch.tail);
    case F32Cfg::kSmall: return plan_cfg<F32Small>(c, name, ch.splits, ch.tail);
    case F32Cfg::kQuad: return plan_cfg<F32Quad>(c, name, ch.splits, ch.tail);
    case F32Cfg::kHalf: return plan_cfg<F32Half>(c, name, ch.splits, ch.tail);
    case F32Cfg::kQuadK: return plan_cfg<F32QuadK>(c, name, ch.splits, ch.tail);
    case F32Cfg::kTinyK: return plan_cfg<F32TinyK>(c, name, ch.splits, ch.tail);
    default: return plan_cfg<F32Tiny>(c, name, ch.splits, ch.tail);
  }
}

static hipError_t launch_f32_as_is(const Call &c) {
  const F32Choice ch = choose_f32(c);
  hipError_t se;
  if (ch.sk > 0) {
    switch (ch.cfg) {
      case F32Cfg::kHuge: if (launch_streamk<F32Huge>(c, ch.sk, &se)) return se; break;
      case F32Cfg::kBig: if (launch_streamk<F32Big>(c, ch.sk, &se)) return se; break;
      case F32Cfg::kMidB: if (launch_streamk<F32MidB>(c, ch.sk, &se)) return se; break;
      case F32Cfg::kQuad: if (launch_streamk<F32Quad>(c, ch.sk, &se)) return se; break;
      case F32Cfg::kHalf: if (launch_streamk<F32Half>(c, ch.sk, &se)) return se; break;
      default: break;
    }
  }
  switch (ch.cfg) {
    case F32Cfg::kHuge: return launch_cfg<F32Huge>(c, ch.splits, ch.tail);
    case F32Cfg::kBig: return launch_cfg<F32Big>(c, ch.splits, ch.tail);
    case F32Cfg::kMid: return launch_cfg<F32Mid>(c, ch.splits, ch.tail);
    case F32Cfg::kMidB: return launch_cfg<F32MidB>(c, ch.splits, ch.tail);
    case F32Cfg::kSmall: return launch_cfg<F32Small>(c, ch.splits, ch.tail);
    case F32Cfg::kQuad: return launch_cfg<F32Quad>(c, ch.splits, ch.tail);
    case F32Cfg::kHalf: return launch_cfg<F32Half>(c, ch.splits, ch.tail);
    case F32Cfg::kQuadK: return launch_cfg<F32QuadK>(c, ch.splits, ch.tail);
    case F32Cfg::kTinyK: return launch_cfg<F32TinyK>(c, ch.splits, ch.tail);
    default: return launch_cfg<F32Tiny>(c, ch.splits, ch.tail);
  }
}

// Operands whose rows do not allow 16-byte loads may first be copied to ones
// that do (pack.hip); the tile and split are then chosen for the copies.
Plan plan_f32(const Call &c) { return plan_packed(c, 4, plan_f32_as_is); }

hipError_t launch_f32(const Call &c) { return run_packed(c, 4, plan_f32_as_is, launch_f32_as_is); }

}  // namespace dgemm
