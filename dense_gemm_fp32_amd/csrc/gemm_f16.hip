// gemm_f16.hip -- fp16-in / fp16-out GEMM with fp32 accumulation on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_f16 for the large tile,
// v_mfma_f32_32x32x16_f16 for the others).
//
// C := alpha*A*B + beta*C with A, B, C in binary16.  Products of halves are
// exact in fp32 and are accumulated in fp32; alpha*acc + beta*C is formed in
// fp32 and rounded once to half, round-to-nearest-even (the fp16 GEMM of the
// "LeetGPU GEMM T4" page: fp32 accumulators, one conversion at the end).
//
// Pipeline.  Each workgroup owns a BM x BN tile of C and walks K in steps of
// BK through STAGES LDS slots (the double buffering of the SGEMM summary's
// tiling section, deepened).  Global tiles move with direct global->LDS loads
// (buffer_load_dwordx4 ... lds: each wave instruction writes 1 KB of LDS
// without passing through registers, from 32-bit per-lane offsets against a
// per-step buffer base); a wave waits for its own loads with an explicit
// vmcnt and a raw barrier publishes the slot, so younger loads stay in flight
// across the barrier.  One barrier per K step, placed before the second half
// of the MFMAs of step kt's last k sub-step, does three things: step kt+1 has
// landed (so its first fragments are read while the last MFMAs of kt run),
// and every wave has read all of step kt's fragments, so step kt's slot is
// refilled at once with step kt+STAGES.  A load thus has STAGES-1 steps of
// compute to arrive, and two slots are enough to run the pipeline.  On the
// eight-wave large tile, half the waves issue all of a step's loads (see
// kSplitLoaders).
//
// LDS layout (per slot, no padding, 16-byte chunks XOR-swizzled by row).
// Each operand keeps its stored orientation (HRegion):
//   * k-major (A as stored, M x K; B stored transposed, N x K): [EXT rows][BK
//     k], row r's logical chunk c at chunk c ^ swz(r), which spreads 8
//     consecutive rows over distinct bank groups for the 128-bit reads.
//   * index-major (B as stored, K x N; A stored transposed, K x M): [BK rows]
//     [EXT], k-row kr's chunk c at c ^ (4*(kr%4) + 2*((kr/8)%2)), so the k-rows
//     read together by a transpose-read pass use distinct banks (four rows
//     for 32x32 blocks, four rows plus the same four 8 rows on for 16x16).
// The swizzle is applied on the global side: lane L of a direct load writes
// LDS bytes 16L..16L+15 of its 1 KB, so it fetches the global chunk that
// belongs there.
//
// Operands.  v_mfma_f32_32x32x16_f16: lane l supplies A(row l%32, k 8h..8h+7)
// and B(k 8h..8h+7, col l%32) for h = l/32; v_mfma_f32_16x16x32_f16 likewise
// with index l%16 and h = l/16 (any k order shared by A and B gives the same
// sum).  With random operands the part holds a higher clock under the 16x16
// form at the same work per clock, so the large tile uses it; its fragments
// cover twice the k, so A is re-read block row by block row into the
// registers just released instead of double-buffered (the whole tile then
// fits 256 VGPRs).  From a k-major region: one ds_read_b128 of the lane's row.
// From an index-major region: two ds_read_b64_tr_b16, each returning 4
// consecutive k of the lane's index from a 4 (k) x 16 (index) block that 16
// lanes address (within each 16-lane group, lane i receives element i%4 of the
// 8-byte rows read by lanes i/4, 4+i/4, 8+i/4, 12+i/4).  The row-major
// product reads A k-major and B index-major; the transposed-operand entry
// points flip either.
//
// Epilogue.  Accumulators leave the MFMA layout (one column per lane) through
// a per-wave LDS staging area, 32 rows at a time (stage_rows); each lane then owns 4
// adjacent columns of a row, reads C there when beta != 0 (8-byte accesses),
// forms alpha*acc + beta*C in fp32, rounds to half and stores 8 bytes, so 32
// lanes write 256 contiguous bytes of a row (the coalesced, LDS-staged
// epilogue of the SGEMM summary).
//
// Edges.  Direct loads cannot substitute zeros, so they are used only where
// every chunk they read lies inside the matrix: rows of a k-major operand
// beyond its extent (M for A, N for B) are clamped to the last row (they only
// feed rows or columns of C that are never stored), chunks of an index-major
// operand beyond its extent are clamped to the last chunk when the extent is
// a multiple of 8.  The partial K step (K % BK != 0) is done first, through
// registers with per-element masks.  A workgroup whose tile crosses the
// extent of an index-major operand that is not a multiple of 8, and every
// workgroup of a call whose A or B is not 16-byte aligned (base or leading
// dimension) or whose offsets would reach 2^31 elements (32-bit load
// offsets), uses the register-staged path instead: masked loads (0 outside
// the matrix; pad elements are never read) written to the same LDS layout.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int STAGES_, int GROUP_M_,
          int MF_ = 32>
struct H16Tile {
  static constexpr int MF = MF_;                       // MFMA block edge: 32x32x16 or 16x16x32
  static constexpr int KM = 512 / MF;                  // k per MFMA
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int STAGES = STAGES_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * kWave;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / MF;
  static constexpr int FN = WTN / MF;
  static constexpr int NG = WTM / 32;                   // 32-row epilogue groups per wave
  static constexpr int SUB = BK / KM;                   // MFMA k sub-steps per K step
  typedef typename std::conditional<MF == 32, f32x16, f32x4>::type Acc;
  static constexpr int ACC_N = MF == 32 ? 16 : 4;
  static constexpr int A_BYTES = BM * BK * 2;           // a slot's A region
  static constexpr int B_BYTES = BK * BN * 2;           // ... and B region
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int QA = A_BYTES / 1024;             // 1 KB wave loads per A tile
  static constexpr int QB = B_BYTES / 1024;
  static constexpr int QA_W = QA / NWAVES;              // ... per wave
  static constexpr int QB_W = QB / NWAVES;
  static constexpr int LOADS = QA_W + QB_W;             // direct loads per wave per K step
  static constexpr int EP_STRIDE = WTN + 4;             // epilogue staging row stride (floats)
  static constexpr int EP_BYTES = 32 * EP_STRIDE * 4;   // per wave
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(BM % (WAVES_M * 32) == 0 && BN % (WAVES_N * 32) == 0, "wave tiling");
  static_assert(BK % 32 == 0 && (SUB % 2 == 0 || MF == 16), "BK multiple of 32");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "1 KB load granules");
  static_assert(QA % NWAVES == 0 && QB % NWAVES == 0, "loads split over waves");
  static_assert(WTM % 64 == 0 && WTN % 64 == 0, "wave origins multiples of 64");
  static_assert(FM % 2 == 0, "the last sub-step splits the block rows in halves");
  static_assert(STAGES >= 2, "the pipeline needs two or more slots");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(NWAVES * EP_BYTES <= LDS_BYTES, "epilogue staging fits in the pipeline LDS");
  static_assert(6 * LOADS <= 63, "vmcnt range");
};

// Operand regions.  A slot holds an A region (BM indices m by BK k) and a B
// region (BN indices n by BK k).  An operand whose memory is k-contiguous (A
// as stored, or B stored transposed, N x K) sits k-contiguous in LDS too:
// rows of 2*BK bytes, one per index ("k-major").  An operand whose memory is
// index-contiguous (B as stored, or A stored transposed, K x M) sits as in
// memory: rows of 2*EXT bytes, one per k ("index-major").  Direct loads copy
// 16-byte chunks, so the LDS orientation follows the memory layout.
//
// Swizzles, chosen from measured gfx950 LDS behaviour: 64 banks of 4 bytes,
// a 128-bit read served 16 lanes (256 bytes) per pass, a 64-bit transpose
// read 32 lanes per pass.
//   k-major: the 16 rows one pass reads must land on 16 distinct 16-byte
//      bank groups of the 256-byte window: row r's chunks are XORed with
//      (r / (256/ROW)) % (ROW/16).
//   index-major: a transpose-read pass covers four k rows x 64 bytes; XORing
//      chunk bits 2-3 with kr % 4 puts the four rows' 64-byte pieces in the
//      four quarters of the window (rows of 128 bytes, two to a window: bit 2
//      with (kr/2) % 2).
template <int EXT, int BK, bool KMAJ>
struct HRegion {
  static constexpr bool K_MAJOR = KMAJ;
  static constexpr int EXTENT = EXT;
  static constexpr int ROW = KMAJ ? 2 * BK : 2 * EXT;      // bytes per LDS row
  static constexpr int CH = ROW / 16;                       // 16-byte chunks per row
  static constexpr int RPW = ROW >= 256 ? 1 : 256 / ROW;    // rows per 256-byte window
  static constexpr int READS = KMAJ ? 1 : 2;                // LDS reads per fragment
  static_assert(KMAJ || ROW >= 128, "index-major rows of at least 128 bytes");
  static_assert(!KMAJ || (32 % RPW == 0 && (32 / RPW) % CH == 0),
                "the swizzle repeats every 32 rows");

  __device__ static __forceinline__ int swz(int row) {
    if constexpr (KMAJ) return (row / RPW) % CH;
    else if constexpr (ROW >= 256) return 4 * (row & 3) + 2 * ((row >> 3) & 1);
    else return 4 * ((row >> 1) & 1);
  }

  // Tile-relative index and k of the 8 elements behind 16-byte chunk
  // (q, lane) of the region (lane L of a 1 KB direct load writes bytes
  // q*1024 + 16L .. +15).
  __device__ static __forceinline__ void chunk(int q, int lane, int &idx, int &kk) {
    const int o = q * 1024 + 16 * lane;
    const int row = o / ROW;
    const int c = ((o % ROW) / 16) ^ swz(row);
    if constexpr (KMAJ) {
      idx = row;
      kk = 8 * c;
    } else {
      kk = row;
      idx = 8 * c;
    }
  }
};

// The two regions of tile T when A is stored transposed (TA) and/or B is
// (TB), and the LDS reads per k sub-step of one wave.
template <class T, bool TA_, bool TB_>
struct HLayout {
  static constexpr bool TA = TA_, TB = TB_;
  typedef HRegion<T::BM, T::BK, !TA_> RA;
  typedef HRegion<T::BN, T::BK, TB_> RB;
  static constexpr int NREAD = T::FM * RA::READS + T::FN * RB::READS;
};

// ---------------------------------------------------------------- direct loads

// This lane's byte offsets, relative to the origin of a K step's tile of the
// operand (the element at index idx0, k k0), of the 16-byte chunks it loads.
// The offsets do not change from step to step; each step only moves the
// buffer base.  They fit in 32 bits when EXT*ld (k-major) or BK*ld
// (index-major) is below 2^31 elements, which the kernel checks before
// taking this path.
template <class T>
struct DirectAddr {
  uint32_t a[2 * T::QA_W];
  uint32_t b[2 * T::QB_W];
};
// Eight-wave 16x16x32 tile: waves 4-7 issue every direct load of a step
// (their own chunks and those of wave - 4) and waves 0-3 none.  A step's 64
// loads take the texture unit longer than a wave's turn at the matrix pipe,
// and a wave whose next load finds the unit's queue full cannot issue its
// MFMAs either; with the loads on one wave per SIMD, the other wave of each
// SIMD never waits at a load (measured: 4096^3 +2%, 8192^3 +2%, bit-identical
// results).
template <class T>
constexpr bool kSplitLoaders = T::MF == 16 && T::NWAVES == 8;

// Offset of the chunk at tile-relative (idx, kk).  Indices past the edge:
// k-major rows are clamped to the last row (they only feed rows or columns of
// C that are never stored); index-major chunks to the last whole chunk
// (ext % 8 == 0 on this path), which also lies inside the matrix.
template <class R>
__device__ __forceinline__ uint32_t direct_offset(int idx, int kk, int idx0, int ext, int ld) {
  int g = idx0 + idx;
  if constexpr (R::K_MAJOR) {
    g = g < ext ? g : ext - 1;
    return 2u * (uint32_t)((g - idx0) * ld + kk);
  } else {
    g = g + 8 <= ext ? g : ext - 8;
    return 2u * (uint32_t)(kk * ld + (g - idx0));
  }
}

// First element of a K step's tile of an operand stored with leading
// dimension ld.
template <class R>
__device__ __forceinline__ const uint16_t *tile_base(const void *X, int idx0, int k0, int ld) {
  const uint16_t *x = static_cast<const uint16_t *>(X);
  return R::K_MAJOR ? x + (size_t)idx0 * (size_t)ld + k0 : x + (size_t)k0 * (size_t)ld + idx0;
}

// The direct path's conditions for one operand: 32-bit offsets, and for an
// index-major operand whose tile crosses the edge, whole chunks up to it.
template <class R, int BK>
__device__ __forceinline__ bool direct_ok(bool edge, int ext, int ld) {
  if constexpr (R::K_MAJOR) return (long long)R::EXTENT * ld < (1LL << 31);
  else return (!edge || (ext % 8) == 0) && (long long)BK * ld < (1LL << 31);
}

template <class T, class L>
__device__ __forceinline__ void direct_setup(const GemmParams &p, int m0, int n0,
                                             DirectAddr<T> &d) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  constexpr int REP = kSplitLoaders<T> ? 2 : 1;
#pragma unroll
  for (int r = 0; r < REP; ++r) {
    const int w = kSplitLoaders<T> ? (r == 0 ? wave - 4 : wave) : wave;
    const int wc = w < 0 ? 0 : w;
#pragma unroll
    for (int j = 0; j < T::QA_W; ++j) {
      int idx, kk;
      L::RA::chunk(wc * T::QA_W + j, lane, idx, kk);
      d.a[r * T::QA_W + j] = direct_offset<typename L::RA>(idx, kk, m0, p.M, p.lda);
    }
#pragma unroll
    for (int j = 0; j < T::QB_W; ++j) {
      int idx, kk;
      L::RB::chunk(wc * T::QB_W + j, lane, idx, kk);
      d.b[r * T::QB_W + j] = direct_offset<typename L::RB>(idx, kk, n0, p.N, p.ldb);
    }
  }
}

template <class T, class L>
__device__ __forceinline__ void direct_issue(const GemmParams &p, const DirectAddr<T> &d, int m0,
                                             int n0, int k0, uint32_t slot_addr) {
  const int wave = wave_id();
  const BufRsrc ra = buffer_rsrc(tile_base<typename L::RA>(p.A, m0, k0, p.lda));
  const BufRsrc rb = buffer_rsrc(tile_base<typename L::RB>(p.B, n0, k0, p.ldb));
  if constexpr (kSplitLoaders<T>) {
    if (wave < 4) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int w = r == 0 ? wave - 4 : wave;
#pragma unroll
      for (int j = 0; j < T::QA_W; ++j)
        buffer_load16(d.a[r * T::QA_W + j], ra, slot_addr + (uint32_t)((w * T::QA_W + j) * 1024));
#pragma unroll
      for (int j = 0; j < T::QB_W; ++j)
        buffer_load16(d.b[r * T::QB_W + j], rb,
                      slot_addr + (uint32_t)(T::A_BYTES + (w * T::QB_W + j) * 1024));
    }
  } else {
#pragma unroll
    for (int j = 0; j < T::QA_W; ++j)
      buffer_load16(d.a[j], ra, slot_addr + (uint32_t)((wave * T::QA_W + j) * 1024));
#pragma unroll
    for (int j = 0; j < T::QB_W; ++j)
      buffer_load16(d.b[j], rb, slot_addr + (uint32_t)(T::A_BYTES + (wave * T::QB_W + j) * 1024));
  }
}

// ---------------------------------------------------------------- register-staged loads

template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t *src) {
  if (VEC) return *reinterpret_cast<const u32x4 *>(src);
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (uint32_t)src[2 * e] | ((uint32_t)src[2 * e + 1] << 16);
  return v;
}

// Eight halves from a 4-byte aligned address as four 4-byte loads (rows whose
// leading dimension is even but not a multiple of 8).
__device__ __forceinline__ u32x4 load8_pairs(const uint16_t *src) {
  const uint32_t *w = reinterpret_cast<const uint32_t *>(src);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// A whole in-range chunk at width w (2 = 16 bytes, 1 = pairs, 0 = elements).
__device__ __forceinline__ u32x4 load8_width(const uint16_t *src, int w) {
  if (w == 2) return load8<true>(src);
  if (w == 1) return load8_pairs(src);
  return load8<false>(src);
}

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

template <class T>
struct RegTile {
  u32x4 a[T::QA_W];
  u32x4 b[T::QB_W];
};

// One chunk of an operand (tile origin idx0, k0) through registers, with 0
// for every element outside the matrix (index >= ext, k >= K).  `w`: the
// operand's load width (its rows start 16-byte aligned: a whole chunk is one
// load; 4-byte aligned: four; otherwise element by element).
template <class R>
__device__ __forceinline__ u32x4 staged_chunk(const void *X, int ld, int idx0, int ext, int k0,
                                              int K, int idx, int kk, int w) {
  const int g = idx0 + idx, gk = k0 + kk;
  if constexpr (R::K_MAJOR) {
    const uint16_t *src = static_cast<const uint16_t *>(X) + (size_t)g * (size_t)ld + gk;
    const bool ok = g < ext;
    if (ok && gk + 7 < K) return load8_width(src, w);
    return load8_masked(src, [&](int e) { return ok && gk + e < K; });
  } else {
    const uint16_t *src = static_cast<const uint16_t *>(X) + (size_t)gk * (size_t)ld + g;
    const bool ok = gk < K;
    if (ok && g + 7 < ext) return load8_width(src, w);
    return load8_masked(src, [&](int e) { return ok && g + e < ext; });
  }
}

// The chunks a direct load would fetch, through registers, with 0 for every
// element outside the matrix (rows >= M, columns >= N, k >= K).
template <class T, class L>
__device__ __forceinline__ void reg_load(const GemmParams &p, int m0, int n0, int k0, int va,
                                         int vb, RegTile<T> &t) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j) {
    int idx, kk;
    L::RA::chunk(wave * T::QA_W + j, lane, idx, kk);
    t.a[j] = staged_chunk<typename L::RA>(p.A, p.lda, m0, p.M, k0, p.K, idx, kk, va);
  }
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j) {
    int idx, kk;
    L::RB::chunk(wave * T::QB_W + j, lane, idx, kk);
    t.b[j] = staged_chunk<typename L::RB>(p.B, p.ldb, n0, p.N, k0, p.K, idx, kk, vb);
  }
}

template <class T>
__device__ __forceinline__ void reg_store(const RegTile<T> &t, char *slot) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < T::QA_W; ++j)
    *reinterpret_cast<u32x4 *>(slot + (wave * T::QA_W + j) * 1024 + 16 * lane) = t.a[j];
#pragma unroll
  for (int j = 0; j < T::QB_W; ++j)
    *reinterpret_cast<u32x4 *>(slot + T::A_BYTES + (wave * T::QB_W + j) * 1024 + 16 * lane) =
        t.b[j];
}

// ---------------------------------------------------------------- fragments and MFMA

template <class T>
struct Frag {
  f16x8 a[T::FM];
  f16x8 b[T::FN];
};

// Per-lane LDS byte offsets of one operand's fragments, relative to its
// region.  k-major: one per k sub-step (block 0; block b adds 32*b rows).
// Index-major: one per block (sub-step 0, first transpose read; sub-step s
// adds 16*s rows).
template <class R, int SUB, int NB>
struct OpAddr {
  int o[R::K_MAJOR ? SUB : NB];
};

template <class T, class L>
struct FragAddr {
  OpAddr<typename L::RA, T::SUB, T::FM> a;
  OpAddr<typename L::RB, T::SUB, T::FN> b;
};

// v_mfma_f32_32x32x16_f16 takes, in lane l, 8 consecutive k (8h..8h+7,
// h = l/32) of index l%32 of the block -- the same shape for A (rows) and B
// (columns).  k-major: one ds_read_b128 of the lane's row.  Index-major: two
// ds_read_b64_tr_b16, each returning 4 consecutive k of the lane's index from
// a 4 (k) x 16 (index) block that 16 lanes address: 16-lane group g reads k
// rows 8*(g/2) + i/4 (+4 for the second read) at indices
// w0 + 32*b + 16*(g%2) + 4*(i%4) .. +3 (i = lane % 16).
template <int MF, class R, int SUB, int NB>
__device__ __forceinline__ void op_setup(int w0, OpAddr<R, SUB, NB> &f) {
  const int lane = threadIdx.x % kWave;
  if constexpr (R::K_MAJOR) {
    // lane l: index l % MF, k group l / MF (8 k each) of the sub-step
    constexpr int G = 64 / MF;
    const int row = w0 + lane % MF, lh = lane / MF;
    const int sw = R::swz(row);
#pragma unroll
    for (int s = 0; s < SUB; ++s) f.o[s] = row * R::ROW + 16 * ((G * s + lh) ^ sw);
  } else if constexpr (MF == 32) {
    const int g = lane / 16, i = lane % 16;
    const int kr = 8 * (g / 2) + i / 4;
    const int t = 2 * (g % 2) + (i % 4) / 2;
    const int sw = R::swz(kr);
#pragma unroll
    for (int b = 0; b < NB; ++b) f.o[b] = kr * R::ROW + 16 * ((w0 / 8 + 4 * b + t) ^ sw) + 8 * (i % 2);
  } else {
    // 16-lane group g reads k rows 8g + i/4 (+4 for the second read) at
    // indices w0 + 16b + 4*(i%4) .. +3: lane i then holds k 8g..8g+7 of index i
    const int g = lane / 16, i = lane % 16;
    const int kr = 8 * g + i / 4;
    const int t = (i % 4) / 2;
    const int sw = R::swz(kr);
#pragma unroll
    for (int b = 0; b < NB; ++b) f.o[b] = kr * R::ROW + 16 * ((w0 / 8 + 2 * b + t) ^ sw) + 8 * (i % 2);
  }
}

template <class T, class L>
__device__ __forceinline__ void frag_setup(int wm0, int wn0, FragAddr<T, L> &f) {
  op_setup<T::MF>(wm0, f.a);
  op_setup<T::MF>(wn0, f.b);
}

// Fragment of block b at k sub-step s from an operand region.
template <int MF, class R, int SUB, int NB>
__device__ __forceinline__ f16x8 op_read(const char *region, const OpAddr<R, SUB, NB> &f, int s,
                                         int b) {
  if constexpr (R::K_MAJOR) {
    return *reinterpret_cast<const f16x8 *>(region + f.o[s] + MF * b * R::ROW);
  } else {
    const char *base = region + f.o[b] + (512 / MF) * s * R::ROW;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + 4 * R::ROW));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// Fragment reads in the order the MFMAs consume them (A block 0, all B
// blocks, then A blocks 1..), so the waits before early MFMAs stay short.
template <class T, class L>
__device__ __forceinline__ void frag_read(const char *slot, const FragAddr<T, L> &f, int s,
                                          Frag<T> &fr) {
  fr.a[0] = op_read<T::MF>(slot, f.a, s, 0);
#pragma unroll
  for (int bj = 0; bj < T::FN; ++bj) fr.b[bj] = op_read<T::MF>(slot + T::A_BYTES, f.b, s, bj);
#pragma unroll
  for (int bi = 1; bi < T::FM; ++bi) fr.a[bi] = op_read<T::MF>(slot, f.a, s, bi);
}

// MFMAs for block rows [BI0, BI1) of one sub-step.
template <class T, int BI0, int BI1>
__device__ __forceinline__ void mfma_rows(const Frag<T> &fr, typename T::Acc (&acc)[T::FM][T::FN]) {
#pragma unroll
  for (int bi = BI0; bi < BI1; ++bi)
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj) {
      if constexpr (T::MF == 32)
        acc[bi][bj] =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(fr.a[bi], fr.b[bj], acc[bi][bj], 0, 0, 0);
      else
        acc[bi][bj] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(fr.a[bi], fr.b[bj], acc[bi][bj], 0, 0, 0);
    }
}

// Scheduling pattern for a region holding NM MFMAs and NR LDS reads: the
// reads are spread evenly behind the first NM - TAIL MFMAs, so they trickle
// into the LDS queue behind MFMAs instead of stalling the wave in front of
// them, and the last of them is issued TAIL MFMAs before the region ends.
template <int I, int NM, int NR, int TAIL>
__device__ __forceinline__ void interleave_slot() {
  if constexpr (I < NM) {
    constexpr int SLOTS = NM - TAIL > 0 ? NM - TAIL : 1;
    constexpr int PER = (NR + SLOTS - 1) / SLOTS;
    constexpr int LEFT = NR - I * PER;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
    if constexpr (I < SLOTS && LEFT > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, LEFT < PER ? LEFT : PER, 0);  // DS reads
    interleave_slot<I + 1, NM, NR, TAIL>();
  }
}

template <int NM, int NR, int TAIL>
__device__ __forceinline__ void interleave_mfma_reads() {
  interleave_slot<0, NM, NR, TAIL>();
}

// Write 32-row group g of a wave's accumulators (rows 32g .. 32g+31 of its
// tile, all its columns) into the wave's staging area, row-major.
template <class T>
__device__ __forceinline__ void stage_rows(float *stage, const typename T::Acc (&acc)[T::FM][T::FN],
                                           int g, int lane) {
  if constexpr (T::MF == 32) {
    const int li = lane % 32, lh = lane / 32;
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage[(8 * (r / 4) + 4 * lh + (r % 4)) * T::EP_STRIDE + 32 * bj + li] = acc[g][bj][r];
  } else {
    // 16x16 block: lane l holds rows 4*(l/16) .. +3 of column l % 16
    const int lc = lane % 16, lq = lane / 16;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stage[(16 * h + 4 * lq + r) * T::EP_STRIDE + 16 * bj + lc] = acc[2 * g + h][bj][r];
  }
}

// ---------------------------------------------------------------- epilogue

template <class T, bool VEC_C, bool CHECK>
__device__ __forceinline__ void epilogue(const GemmParams &p, int r0, int c0, char *lds,
                                         const typename T::Acc (&acc)[T::FM][T::FN]) {
  uint16_t *C = static_cast<uint16_t *>(p.C);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  float *stage = reinterpret_cast<float *>(lds + wave * T::EP_BYTES);
  const float alpha = p.alpha, beta = p.beta;
  constexpr int LPR = T::WTN / 4;                 // lanes per staged row
  constexpr int ROWS_PER_PASS = kWave / LPR;
  constexpr int PASSES = 32 / ROWS_PER_PASS;
  const int cl = 4 * (lane % LPR);
  const int col = c0 + cl;
  const bool cols_ok = !CHECK || col + 3 < p.N;
  // C values are loaded ahead of their use, so the latencies of the loads
  // overlap instead of adding up pass by pass (a store to C keeps a later
  // load of C from moving above it).  Vector C: every value this lane
  // combines, before the first block row is staged (8-byte loads; the lanes
  // past an edge tile's last full group of 4 columns load theirs when they
  // store).  Element-wise C: one block row at a time, masked at the matrix
  // edge, which is what the registers of the largest tile allow; values are
  // packed two halves per word.
  u32x2 cpre[VEC_C ? T::NG : 1][PASSES];
  if (VEC_C && beta != 0.0f) {
#pragma unroll
    for (int bi = 0; bi < T::NG; ++bi)
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int row = r0 + 32 * bi + pass * ROWS_PER_PASS + lane / LPR;
        cpre[VEC_C ? bi : 0][pass] = u32x2{0u, 0u};
        if (!CHECK || (row < p.M && cols_ok))
          cpre[VEC_C ? bi : 0][pass] =
              *reinterpret_cast<const u32x2 *>(C + (size_t)row * (size_t)p.ldc + col);
      }
  }
#pragma unroll
  for (int bi = 0; bi < T::NG; ++bi) {
    if (!VEC_C && beta != 0.0f) {
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int row = r0 + 32 * bi + pass * ROWS_PER_PASS + lane / LPR;
        const uint16_t *src = C + (size_t)row * (size_t)p.ldc + col;
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = (!CHECK || (row < p.M && col + e < p.N)) ? (uint32_t)src[e] : 0u;
        cpre[0][pass] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      }
    }
    stage_rows<T>(stage, acc, bi, lane);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rl = pass * ROWS_PER_PASS + lane / LPR;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&stage[rl * T::EP_STRIDE + cl]);
      const int row = r0 + 32 * bi + rl;
      if (CHECK && row >= p.M) continue;
      uint16_t *dst = C + (size_t)row * (size_t)p.ldc + col;
      if (VEC_C && cols_ok) {
        float o[4];
        if (beta != 0.0f) {
          const u32x2 w = cpre[VEC_C ? bi : 0][pass];
          o[0] = __builtin_fmaf(beta, f16_bits_to_f32((uint16_t)(w[0] & 0xffff)), alpha * v[0]);
          o[1] = __builtin_fmaf(beta, f16_bits_to_f32((uint16_t)(w[0] >> 16)), alpha * v[1]);
          o[2] = __builtin_fmaf(beta, f16_bits_to_f32((uint16_t)(w[1] & 0xffff)), alpha * v[2]);
          o[3] = __builtin_fmaf(beta, f16_bits_to_f32((uint16_t)(w[1] >> 16)), alpha * v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = alpha * v[e];
        }
        u32x2 ow;
        ow[0] = (uint32_t)f32_to_f16_bits(o[0]) | ((uint32_t)f32_to_f16_bits(o[1]) << 16);
        ow[1] = (uint32_t)f32_to_f16_bits(o[2]) | ((uint32_t)f32_to_f16_bits(o[3]) << 16);
        *reinterpret_cast<u32x2 *>(dst) = ow;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (CHECK && col + e >= p.N) continue;
          float o = alpha * v[e];
          if (beta != 0.0f) {
            const u32x2 w = cpre[0][pass];
            const uint16_t ce =
                VEC_C ? dst[e] : (uint16_t)((e < 2 ? w[0] : w[1]) >> (16 * (e & 1)));
            o = __builtin_fmaf(beta, f16_bits_to_f32(ce), o);
          }
          dst[e] = f32_to_f16_bits(o);
        }
      }
    }
  }
}

// The same epilogue for an fp32 C and result: alpha*acc + beta*C in fp32,
// written as 16-byte stores (4 adjacent floats per lane, 512 contiguous
// bytes per 32 lanes).  C is loaded one block row at a time (16-byte loads,
// or element by element, masked, where C does not allow them), before that
// row's accumulators are staged, so the load latency overlaps the staging
// without holding every row's C in registers at once.
template <class T, bool VEC_C, bool CHECK>
__device__ __forceinline__ void epilogue_out32(const GemmParams &p, int r0, int c0, char *lds,
                                               const typename T::Acc (&acc)[T::FM][T::FN]) {
  float *C = static_cast<float *>(p.C);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  float *stage = reinterpret_cast<float *>(lds + wave * T::EP_BYTES);
  const float alpha = p.alpha, beta = p.beta;
  constexpr int LPR = T::WTN / 4;
  constexpr int ROWS_PER_PASS = kWave / LPR;
  constexpr int PASSES = 32 / ROWS_PER_PASS;
  const int cl = 4 * (lane % LPR);
  const int col = c0 + cl;
  const bool cols_ok = !CHECK || col + 3 < p.N;
#pragma unroll
  for (int bi = 0; bi < T::NG; ++bi) {
    f32x4 cpre[PASSES];
    if (beta != 0.0f) {
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int row = r0 + 32 * bi + pass * ROWS_PER_PASS + lane / LPR;
        const float *src = C + (size_t)row * (size_t)p.ldc + col;
        cpre[pass] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (VEC_C) {
          if (!CHECK || (row < p.M && cols_ok)) cpre[pass] = *reinterpret_cast<const f32x4 *>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!CHECK || (row < p.M && col + e < p.N)) cpre[pass][e] = src[e];
        }
      }
    }
    stage_rows<T>(stage, acc, bi, lane);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rl = pass * ROWS_PER_PASS + lane / LPR;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&stage[rl * T::EP_STRIDE + cl]);
      const int row = r0 + 32 * bi + rl;
      if (CHECK && row >= p.M) continue;
      float *dst = C + (size_t)row * (size_t)p.ldc + col;
      if (VEC_C && cols_ok) {
        f32x4 o;
        if (beta != 0.0f) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(beta, cpre[pass][e], alpha * v[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = alpha * v[e];
        }
        *reinterpret_cast<f32x4 *>(dst) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (CHECK && col + e >= p.N) continue;
          float o = alpha * v[e];
          if (beta != 0.0f) o = __builtin_fmaf(beta, VEC_C ? dst[e] : cpre[pass][e], o);
          dst[e] = o;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- main loops

template <class T>
__device__ __forceinline__ void zero_acc(typename T::Acc (&acc)[T::FM][T::FN]) {
#pragma unroll
  for (int bi = 0; bi < T::FM; ++bi)
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj)
#pragma unroll
      for (int r = 0; r < T::ACC_N; ++r) acc[bi][bj][r] = 0.0f;
}

// All sub-steps of one K step from LDS slot `slot`.  On entry fr[0] holds
// sub-step 0.  Each sub-step's MFMAs run interleaved with the reads of the
// next sub-step's fragments.  In the last sub-step the first half of the MFMAs
// is issued, then `next()` publishes the following slot (its barrier wait
// overlaps those MFMAs) and may issue loads, then sub-step 0 of the following
// K step is read from `next_slot` into fr[0] between the remaining MFMAs.  On
// the last K step this reads a stale slot whose values are never used:
// keeping the reads unconditional keeps the LDS wait counts exact.
//
// kstep_rolling is that schedule for 16x16x32 blocks, whose sub-step
// fragments take twice the registers of the 32x32x16 ones, too many to
// double-buffer: on entry fr holds sub-step 0; A is read block row by block
// row into the registers the row's MFMAs just released, and only B has a
// second buffer (bn).  kstep picks the schedule by the tile's block shape.
template <class T, class L, class Next>
__device__ __forceinline__ void kstep_rolling(const char *slot, const char *next_slot,
                                              const FragAddr<T, L> &fa, Frag<T> &fr,
                                              typename T::Acc (&acc)[T::FM][T::FN], Next next) {
  constexpr int HALF = T::FM / 2;
#pragma unroll
  for (int s = 0; s < T::SUB; ++s) {
    f16x8 bn[T::FN];
    if (s + 1 < T::SUB) {
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj) bn[bj] = op_read<T::MF>(slot + T::A_BYTES, fa.b, s + 1, bj);
#pragma unroll
      for (int bi = 0; bi < T::FM; ++bi) {
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj)
          acc[bi][bj] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(fr.a[bi], fr.b[bj], acc[bi][bj], 0, 0, 0);
        fr.a[bi] = op_read<T::MF>(slot, fa.a, s + 1, bi);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int bi = 0; bi < HALF; ++bi)
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj)
          acc[bi][bj] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(fr.a[bi], fr.b[bj], acc[bi][bj], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      next();
#pragma unroll
      for (int bj = 0; bj < T::FN; ++bj) bn[bj] = op_read<T::MF>(next_slot + T::A_BYTES, fa.b, 0, bj);
#pragma unroll
      for (int bi = 0; bi < HALF; ++bi) fr.a[bi] = op_read<T::MF>(next_slot, fa.a, 0, bi);
#pragma unroll
      for (int bi = HALF; bi < T::FM; ++bi) {
#pragma unroll
        for (int bj = 0; bj < T::FN; ++bj)
          acc[bi][bj] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(fr.a[bi], fr.b[bj], acc[bi][bj], 0, 0, 0);
        fr.a[bi] = op_read<T::MF>(next_slot, fa.a, 0, bi);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bj = 0; bj < T::FN; ++bj) fr.b[bj] = bn[bj];
  }
}

template <class T, class L, class Next>
__device__ __forceinline__ void kstep(const char *slot, const char *next_slot,
                                      const FragAddr<T, L> &fa, Frag<T> (&fr)[2],
                                      typename T::Acc (&acc)[T::FM][T::FN], Next next) {
  if constexpr (T::MF == 16) {
    kstep_rolling<T, L>(slot, next_slot, fa, fr[0], acc, next);   // fr[1] is not used
  } else {
    constexpr int NREAD = L::NREAD;     // LDS instructions per sub-step
    constexpr int HALF = T::FM / 2;
#pragma unroll
    for (int s = 0; s < T::SUB; ++s) {
      if (s + 1 < T::SUB) {
        frag_read<T, L>(slot, fa, s + 1, fr[(s + 1) & 1]);
        mfma_rows<T, 0, T::FM>(fr[s & 1], acc);
        interleave_mfma_reads<T::FM * T::FN, NREAD, 4>();
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mfma_rows<T, 0, HALF>(fr[s & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
        next();
        frag_read<T, L>(next_slot, fa, 0, fr[0]);
        mfma_rows<T, HALF, T::FM>(fr[s & 1], acc);
        interleave_mfma_reads<(T::FM - HALF) * T::FN, NREAD, 2>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Direct-load pipeline over STAGES slots: slot j % STAGES holds step j.
template <class T, class L>
__device__ __forceinline__ void mainloop_direct(const GemmParams &p, int m0, int n0, char *lds,
                                                uint32_t lds_u32, int wm0, int wn0,
                                                typename T::Acc (&acc)[T::FM][T::FN]) {
  const KSteps ks = make_steps(p.K, T::BK);
  DirectAddr<T> da;
  direct_setup<T, L>(p, m0, n0, da);
  FragAddr<T, L> fa;
  frag_setup<T, L>(wm0, wn0, fa);

  // Prologue: step 0 (masked, through registers, when it is the partial
  // step), then direct loads of steps 1 .. STAGES-1.
  if (ks.tail) {
    RegTile<T> t;
    reg_load<T, L>(p, m0, n0, ks.k0(0), 2, 2, t);
    reg_store<T>(t, lds);
  } else {
    direct_issue<T, L>(p, da, m0, n0, ks.k0(0), lds_u32);
  }
  int issued = 1;
#pragma unroll
  for (int j = 1; j < T::STAGES; ++j) {
    if (j < ks.nk) {
      direct_issue<T, L>(p, da, m0, n0, ks.k0(j), lds_u32 + (uint32_t)(j * T::STAGE_BYTES));
      ++issued;
    }
  }
  // Publish step 0; the loads of steps 1.. may stay in flight.
  constexpr int WL = kSplitLoaders<T> ? 2 * T::LOADS : T::LOADS;
  wait_direct<WL>(issued - 1);
  lds_barrier();

  Frag<T> fr[2];
  frag_read<T, L>(lds, fa, 0, fr[0]);

  for (int kt = 0; kt < ks.nk; ++kt) {
    const int slot_no = kt % T::STAGES;
    const char *slot = lds + slot_no * T::STAGE_BYTES;
    const char *next_slot = lds + ((kt + 1) % T::STAGES) * T::STAGE_BYTES;
    kstep<T, L>(slot, next_slot, fa, fr, acc, [&]() {
      // Step kt+1 must have landed (steps issued after it may stay in
      // flight), and this wave's reads of step kt must be complete.  After
      // the last step nothing is in flight and this is a full wait.
      wait_direct<WL>((issued - 1) - (kt + 1));
      lds_barrier();
      // Every wave has read all of step kt: its slot takes step kt+STAGES.
      const int nx = kt + T::STAGES;
      if (nx < ks.nk) {
        direct_issue<T, L>(p, da, m0, n0, ks.k0(nx), lds_u32 + (uint32_t)(slot_no * T::STAGE_BYTES));
        ++issued;
      }
    });
  }
}

// Register-staged double-buffered pipeline (unaligned operands, ragged
// edges of index-major operands).
template <class T, class L>
__device__ __forceinline__ void mainloop_staged(const GemmParams &p, int m0, int n0, char *lds,
                                                int wm0, int wn0, int va, int vb,
                                                typename T::Acc (&acc)[T::FM][T::FN]) {
  const KSteps ks = make_steps(p.K, T::BK);
  FragAddr<T, L> fa;
  frag_setup<T, L>(wm0, wn0, fa);
  RegTile<T> t;
  reg_load<T, L>(p, m0, n0, ks.k0(0), va, vb, t);
  reg_store<T>(t, lds);
  __syncthreads();
  Frag<T> fr[2];
  frag_read<T, L>(lds, fa, 0, fr[0]);
  for (int kt = 0; kt < ks.nk; ++kt) {
    const char *slot = lds + (kt % 2) * T::STAGE_BYTES;
    char *nslot = lds + ((kt + 1) % 2) * T::STAGE_BYTES;
    if (kt + 1 < ks.nk) reg_load<T, L>(p, m0, n0, ks.k0(kt + 1), va, vb, t);
    // nslot was last read in step kt-1, before that step's barrier.  On the
    // last step the store repeats old data into a slot nobody reads again.
    kstep<T, L>(slot, nslot, fa, fr, acc, [&]() {
      reg_store<T>(t, nslot);
      __syncthreads();
    });
  }
}

// TA / TB: A is stored transposed (K x M, lda >= M) / B is (N x K, ldb >= K).
// OUT32: C and the result are fp32 (fp16 inputs); otherwise fp16.
template <class T, bool TA, bool TB, bool VC, bool OUT32>
__global__ __launch_bounds__(T::NT) void hgemm_mfma(GemmParams p) {
  typedef HLayout<T, TA, TB> L;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];
  lds_poison(lds, T::LDS_BYTES);
  int tm, tn, split;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
  select_split<uint16_t, float, TA, TB>(p, split);   // split-K passes always write fp32 slabs
  const int m0 = tm * T::BM;
  const int n0 = tn * T::BN;
  const int wave = threadIdx.x / kWave;
  const int wm0 = (wave / T::WAVES_N) * T::WTM;
  const int wn0 = (wave % T::WAVES_N) * T::WTN;
  typename T::Acc acc[T::FM][T::FN];
  zero_acc<T>(acc);

  const bool m_edge = m0 + T::BM > p.M;
  const bool n_edge = n0 + T::BN > p.N;
  const int va = vec_width_a(p.vec_ab), vb = vec_width_b(p.vec_ab);
  const bool direct = va == 2 && vb == 2 && direct_ok<typename L::RA, T::BK>(m_edge, p.M, p.lda) &&
                      direct_ok<typename L::RB, T::BK>(n_edge, p.N, p.ldb);
  if (direct) mainloop_direct<T, L>(p, m0, n0, lds, lds_address(lds), wm0, wn0, acc);
  else mainloop_staged<T, L>(p, m0, n0, lds, wm0, wn0, va, vb, acc);

  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();   // every wave is done with the pipeline slots
  const bool edge = n_edge || m_edge;
  if constexpr (OUT32) {
    if (edge) epilogue_out32<T, VC, true>(p, m0 + wm0, n0 + wn0, lds, acc);
    else epilogue_out32<T, VC, false>(p, m0 + wm0, n0 + wn0, lds, acc);
  } else {
    if (edge) epilogue<T, VC, true>(p, m0 + wm0, n0 + wn0, lds, acc);
    else epilogue<T, VC, false>(p, m0 + wm0, n0 + wn0, lds, acc);
  }
}

// ---------------------------------------------------------------- host side

// Tile configurations (BM, BN, BK, waves along M, waves along N, LDS slots,
// L2 group rows), largest first; a call takes the largest tile that still
// gives at least half of the CUs a workgroup.
typedef H16Tile<256, 256, 64, 2, 4, 2, 4, 16> F16Big;     // 8 waves, 128 KB LDS, 1 WG/CU, 16x16x32
typedef H16Tile<256, 256, 64, 2, 4, 2, 4, 32> F16Big32;   // the same tile on 32x32x16 blocks
typedef H16Tile<128, 128, 32, 2, 2, 4, 8> F16Mid;     // 4 waves,  64 KB LDS, 2 WG/CU
typedef H16Tile<64, 128, 32, 1, 2, 4, 8> F16Small;    // 2 waves,  48 KB LDS, 3 WG/CU

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
  // element pairs (4 bytes) when a leading dimension is even but 16-byte
  // loads are out
  const bool pa = !va && !c.force_scalar && vec_ok(c.A, c.lda, 2);
  const bool pb = !vb && !c.force_scalar && vec_ok(c.B, c.ldb, 2);
  // C: 4 adjacent elements per access (8 bytes of fp16 or 16 of fp32).
  const bool vc = !c.force_scalar && (c.ldc % 4) == 0 &&
                  aligned_to(c.C, (uintptr_t)(c.out32 ? 16 : 8));
  pl.vec_a = va ? 8 : (pa ? 2 : 1);
  pl.vec_b = vb ? 8 : (pb ? 2 : 1);
  pl.vec_c = vc ? 4 : 1;
  const long long tm = (c.M + T::BM - 1) / T::BM;
  const long long tn = (c.N + T::BN - 1) / T::BN;
  pl.blocks = tm * tn;
  pl.splits = 1;
  pl.tail = 1;
  pl.ws_bytes = 0;
  return pl;
}

template <class T, bool TA, bool TB, bool VC, bool OUT32>
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
  p.splits = c.splits;
  p.k_chunk = c.k_chunk;
  p.split_stride = c.split_stride;
  p.vec_ab = vec_bits(pl.vec_a, pl.vec_b, 8);
  p.tile_base = 0;
  p.tile_count = 0;
  p.c_tiles = 0;
  hipLaunchKernelGGL((hgemm_mfma<T, TA, TB, VC, OUT32>), dim3((unsigned)(pl.blocks * c.splits)),
                     dim3(T::NT), 0, c.stream, p);
  return hipGetLastError();
}

template <class T, bool OUT32>
static hipError_t dispatch_out(const Call &c, const Plan &pl) {
  const int key = (c.ta ? 4 : 0) | (c.tb ? 2 : 0) | (pl.vec_c > 1 ? 1 : 0);
  switch (key) {
    case 0: return launch_variant<T, false, false, false, OUT32>(c, pl);
    case 1: return launch_variant<T, false, false, true, OUT32>(c, pl);
    case 2: return launch_variant<T, false, true, false, OUT32>(c, pl);
    case 3: return launch_variant<T, false, true, true, OUT32>(c, pl);
    case 4: return launch_variant<T, true, false, false, OUT32>(c, pl);
    case 5: return launch_variant<T, true, false, true, OUT32>(c, pl);
    default: break;
  }
  // Both operands stored transposed: with 16x16x32 blocks that kernel needs
  // more than 256 VGPRs (it spills), so it keeps the 32x32x16 blocks.
  typedef typename std::conditional<
      T::MF == 16,
      H16Tile<T::BM, T::BN, T::BK, T::WAVES_M, T::WAVES_N, T::STAGES, T::GROUP_M, 32>, T>::type TT;
  if (key == 6) return launch_variant<TT, true, true, false, OUT32>(c, pl);
  return launch_variant<TT, true, true, true, OUT32>(c, pl);
}

template <class T>
static hipError_t dispatch(const Call &c) {
  const Plan pl = make_plan<T>(c, "");
  if (pl.blocks * c.splits > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  return c.out32 ? dispatch_out<T, true>(c, pl) : dispatch_out<T, false>(c, pl);
}

template <class T>
static long long tiles_of(const Call &c) {
  return (long long)((c.M + T::BM - 1) / T::BM) * (long long)((c.N + T::BN - 1) / T::BN);
}

enum class F16Cfg { kBig, kBig32, kMid, kSmall };

// Share of the CUs kept busy by `tiles` workgroups (whole tiles per CU) and
// share of the two-waves-per-SIMD occupancy a busy CU reaches with its
// resident workgroups (one wave per SIMD leaves the matrix pipe idle while
// the wave waits: measured, the 128x128 tile runs 2x faster per CU with two
// workgroups resident than with one).
static double busy_share16(long long tiles) {
  const double per_cu = (double)tiles / kCUs;
  const double rounds = (double)((tiles + kCUs - 1) / kCUs);
  return per_cu / rounds;
}

template <class T>
static double score16(const Call &c, double eff, int per_cu, int splits) {
  const long long t = tiles_of<T>(c) * splits;
  long long resident = (t + kCUs - 1) / kCUs;
  if (resident > per_cu) resident = per_cu;
  const double waves = (double)(resident * T::NWAVES);
  return eff * busy_share16(t) * (waves >= 8.0 ? 1.0 : waves / 8.0);
}

struct F16Choice {
  F16Cfg cfg;
  int splits;
  double time;   // estimated seconds
};

// Estimated time: the product at `score` of the fp16 peak, plus, when K is
// split S ways, the extra pass (launch, and S fp32 slabs of M x N written and
// read back at ~6 TB/s; the writes overlap the product).
static double est_time16(const Call &c, double score, int splits) {
  const double flops = 2.0 * (double)c.M * (double)c.N * (double)c.K;
  double t = flops / (score * 2516.6e12);
  if (splits > 1) t += 4e-6 + 8.0 * splits * (double)c.M * (double)c.N / 6e12;
  return t;
}

template <class T>
static void try_splits16(const Call &c, F16Cfg cfg, double eff, int per_cu, F16Choice &best) {
  for (int S = 2; S <= 8; ++S) {
    const int kc = ((c.K + S - 1) / S + T::BK - 1) / T::BK * T::BK;
    if (kc < 1024) break;
    const int used = (c.K + kc - 1) / kc;
    const double t = est_time16(c, score16<T>(c, eff, per_cu, used), used);
    if (t < best.time * 0.98) best = F16Choice{cfg, used, t};
  }
}

// Unsplit: measured, the large tile stays ahead down to about half a round
// of tiles (fewer busy CUs draw less power and clock higher), the medium one
// down to half a round as well.  K is split only when it is at least twice
// max(M, N): the fp16 product is fast enough that the extra pass over the
// fp32 slabs pays only for deep K (512 x 512 x 8192 and 1024 x 1024 x 8192:
// 2-3x with 8 chunks of the 128x128 tile; no square size gains).  Scores use
// the tiles' throughput at two waves per SIMD as a fraction of the fp16 peak
// (0.47, 0.47, 0.42); split candidates' chunks are at least 1024 deep and
// the fastest estimate (est_time16) wins.
// Calls with an operand that cannot take 16-byte loads run the element-wise
// staged loads, and their workgroups need company on the CU to hide them.
// Measured (interleaved, every tile and split of 1-4) on six such shapes with
// fewer than 1.5 medium tiles per CU, the best was always the 128x128 tile
// with the smallest K split reaching 1.5 workgroups per CU (at most 4, chunks
// of at least 128 k): 1000x3000x517 86.6 against 83.7 TFLOP/s for the
// direct-path choice, 2000x2000x1000 165 / 152, 1500^3 119 / 67,
// 517x3000x1000 91 / 54, 1000x1000x4000 unchanged.  (The element-wise load
// test switch does not count: it never changes the tile or the split.)
static bool staged_call16(const Call &c) {
  return !vec_ok(c.A, c.lda, 8) || !vec_ok(c.B, c.ldb, 8);
}

static F16Choice choose_f16(const Call &c) {
  const int forced = c.split_mode >= 2 ? c.split_mode : 1;
  if (c.tile_config == 1) return F16Choice{F16Cfg::kBig, forced, 0.0};
  if (c.tile_config == 6) return F16Choice{F16Cfg::kBig32, forced, 0.0};
  if (c.tile_config == 2 || c.tile_config == 5) return F16Choice{F16Cfg::kMid, forced, 0.0};
  if (c.tile_config == 3 || c.tile_config == 4 || c.tile_config == 7 || c.tile_config >= 9)
    return F16Choice{F16Cfg::kSmall, forced, 0.0};
  if (c.tile_config == 8) return F16Choice{F16Cfg::kMid, forced, 0.0};
  const long long mid_tiles = tiles_of<F16Mid>(c);
  if (c.split_mode == 0 && staged_call16(c) && 2 * mid_tiles < 3LL * kCUs &&
      tiles_of<F16Small>(c) >= kCUs / 2) {
    int S = 1;
    while (S < 4 && 2 * mid_tiles * S < 3LL * kCUs &&
           ((c.K + S) / (S + 1) + F16Mid::BK - 1) / F16Mid::BK * F16Mid::BK >= 128)
      ++S;
    return F16Choice{F16Cfg::kMid, S, 0.0};
  }
  F16Choice best;
  if (tiles_of<F16Big>(c) >= kCUs / 2)
    best = F16Choice{F16Cfg::kBig, 1, est_time16(c, score16<F16Big>(c, 0.47, 1, 1), 1)};
  else if (tiles_of<F16Mid>(c) >= kCUs / 2)
    best = F16Choice{F16Cfg::kMid, 1, est_time16(c, score16<F16Mid>(c, 0.47, 2, 1), 1)};
  else
    best = F16Choice{F16Cfg::kSmall, 1, est_time16(c, score16<F16Small>(c, 0.42, 3, 1), 1)};
  if (c.split_mode == 0 && c.K >= 2 * (c.M > c.N ? c.M : c.N)) {
    try_splits16<F16Big>(c, F16Cfg::kBig, 0.47, 1, best);
    try_splits16<F16Mid>(c, F16Cfg::kMid, 0.47, 2, best);
    try_splits16<F16Small>(c, F16Cfg::kSmall, 0.42, 3, best);
  } else if (c.split_mode >= 2) {
    best.splits = forced;
  }
  // The large tile's two block shapes.  16x16x32 blocks let the part hold a
  // higher clock where it is power-bound, but do a little less work per clock
  // (A re-read per block row): they win when the workgroups fill at least
  // three quarters of the CUs and the clock drops (interleaved, sustained:
  // 4096^3 +3.5-6%, 5120^3 +2.7%, 8192^3 +2.7%; 196 tiles, 3456^3 and
  // 3584^3: +4%, 225 tiles, 3712^3 and 3840^3: +5%, 3584x3584x8192 +5%) and
  // lose where more of the chip idles and the clock stays near its maximum
  // (144 tiles, 3072^3: -2 to -7.5%; 128 and 160 tiles: -1 to -4%; 169: even).
  if (best.cfg == F16Cfg::kBig && 4 * tiles_of<F16Big>(c) * best.splits < 3LL * kCUs)
    best.cfg = F16Cfg::kBig32;
  return best;
}

// Run configuration T, splitting K when the split count says so: the tiles
// of every K chunk write raw fp32 sums (the fp32-output kernel) to a pooled
// workspace, then one pass sums the chunks in order, applies alpha and beta
// and rounds to C's type.  If the workspace cannot be had the call runs
// unsplit.
template <class T>
static hipError_t launch_cfg(const Call &c, int want) {
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
  pc.out32 = true;
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
    r.half_out = !c.out32;
    r.force_scalar = c.force_scalar;
    e = launch_splitk_reduce(r, c.stream);
  }
  const hipError_t f = workspace_free(c, ws);
  return e != hipSuccess ? e : f;
}

template <class T>
static Plan plan_cfg(const Call &c, const char *name, int want) {
  Plan pl = make_plan<T>(c, name);
  int kc = 0;
  pl.splits = clamp_splits(c, want, T::BK, pl.blocks, &kc);
  pl.ws_bytes = pl.splits > 1 ? split_ws_bytes(pl.splits, c.M, c.N) : 0;
  return pl;
}

static Plan plan_f16_as_is(const Call &c) {
  const F16Choice ch = choose_f16(c);
  switch (ch.cfg) {
    case F16Cfg::kBig:
      if (c.ta && c.tb)   // both operands transposed: 32x32x16 blocks (see dispatch_out)
        return plan_cfg<F16Big>(c, c.out32 ? "f16 mfma32x32x16 tile 256x256x64 8 waves 2 slots out f32"
                                           : "f16 mfma32x32x16 tile 256x256x64 8 waves 2 slots",
                                ch.splits);
      return plan_cfg<F16Big>(c, c.out32 ? "f16 mfma16x16x32 tile 256x256x64 8 waves 2 slots out f32"
                                         : "f16 mfma16x16x32 tile 256x256x64 8 waves 2 slots", ch.splits);
    case F16Cfg::kBig32:
      return plan_cfg<F16Big32>(c, c.out32 ? "f16 mfma32x32x16 tile 256x256x64 8 waves 2 slots out f32"
                                           : "f16 mfma32x32x16 tile 256x256x64 8 waves 2 slots",
                                ch.splits);
    case F16Cfg::kMid:
      return plan_cfg<F16Mid>(c, c.out32 ? "f16 mfma32x32x16 tile 128x128x32 4 waves 4 slots out f32"
                                         : "f16 mfma32x32x16 tile 128x128x32 4 waves 4 slots", ch.splits);
    default:
      return plan_cfg<F16Small>(c, c.out32 ? "f16 mfma32x32x16 tile 64x128x32 2 waves 4 slots out f32"
                                           : "f16 mfma32x32x16 tile 64x128x32 2 waves 4 slots", ch.splits);
  }
}

static hipError_t launch_f16_as_is(const Call &c) {
  const F16Choice ch = choose_f16(c);
  switch (ch.cfg) {
    case F16Cfg::kBig: return launch_cfg<F16Big>(c, ch.splits);
    case F16Cfg::kBig32: return launch_cfg<F16Big32>(c, ch.splits);
    case F16Cfg::kMid: return launch_cfg<F16Mid>(c, ch.splits);
    default: return launch_cfg<F16Small>(c, ch.splits);
  }
}

// Operands whose rows do not allow 16-byte loads may first be copied to ones
// that do (pack.hip); the tile and split are then chosen for the copies.
Plan plan_f16(const Call &c) { return plan_packed(c, 2, plan_f16_as_is); }

hipError_t launch_f16(const Call &c) { return run_packed(c, 2, plan_f16_as_is, launch_f16_as_is); }

}  // namespace dgemm
