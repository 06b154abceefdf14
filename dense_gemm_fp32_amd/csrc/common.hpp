// common.hpp -- shared device-side definitions of the gfx950 GEMM kernels.
//
// Layout convention everywhere: row-major, element (i, j) of a matrix with
// leading dimension ld at ptr[i*ld + j] (the SGEMM summary's memory-layout
// section).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kXcds = 8;        // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kCUs = 256;       // MI355X compute units (tile-size choice)

// Kernel arguments (passed by value; lives in the kernarg segment).
struct GemmParams {
  const void *A;
  const void *B;
  void *C;
  int M, N, K;
  int lda, ldb, ldc;
  float alpha, beta;
  int tiles_m, tiles_n;   // ceil(M/BM), ceil(N/BN)
  int group_m;            // tile rows per L2 group
  // Split K: `splits` > 1 divides K into chunks of k_chunk (a multiple of
  // the tile's K step; the last chunk takes the rest).  Workgroup (tile,
  // split s) multiplies A(:, chunk s) by B(chunk s, :) and writes the raw fp32
  // sums to C + s*split_stride (a workspace, ldc its row pitch); the caller
  // sets alpha = 1, beta = 0 for that pass and reduces the slabs afterwards.
  int splits;
  int k_chunk;
  long long split_stride;  // elements between the slabs of consecutive splits
  // Bit 0: every row of A starts 16-byte aligned (vector loads); bit 1: of B.
  // Bit 2: every row of A starts aligned to two elements (the register-staged
  // path loads element pairs: 8 bytes of fp32, 4 of fp16); bit 3: of B.
  int vec_ab;
  // A launch may cover part of the tile order: tiles [tile_base, tile_base +
  // tile_count) of the grouped order (tile_count 0: all of them).  With
  // c_tiles set, a split-K pass writes each (split, tile) result as a dense
  // BM x BN fp32 block at C + (split*tile_count + local tile)*BM*BN instead
  // of into an M x N slab.
  int tile_base, tile_count;
  int c_tiles;
};

// A Stream-K launch: the first `dp` workgroups each compute one of tiles
// 0 .. dp-1 whole; the K steps of the other tiles (dp .. tiles-1, `steps`
// each) are dealt out in runs of `iters` steps to the remaining workgroups.
// W holds two BM x BN fp32 blocks per such workgroup for the parts of tiles
// it covers.
struct StreamKRun {
  int tiles, steps, dp;
  long long iters;
  float *W;
};

// Restrict the kernel arguments to split `s` of a split-K launch: K range
// [s*k_chunk, min(K, (s+1)*k_chunk)) and that split's output slab.  TA / TB:
// A is stored K x M / B is stored N x K (k runs along the rows).
template <typename TIn, typename TOut, bool TA = false, bool TB = false>
__device__ __forceinline__ void select_split(GemmParams &p, int s) {
  if (p.splits <= 1) return;
  const int kb = s * p.k_chunk;
  const int left = p.K - kb;
  p.K = left < p.k_chunk ? left : p.k_chunk;
  p.A = static_cast<const TIn *>(p.A) + (TA ? (size_t)kb * (size_t)p.lda : (size_t)kb);
  p.B = static_cast<const TIn *>(p.B) + (TB ? (size_t)kb : (size_t)kb * (size_t)p.ldb);
  p.C = static_cast<TOut *>(p.C) + (size_t)s * (size_t)p.split_stride;
}

// Tile (tm, tn) at position b of the grouped order (see tile_of_block).
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int group_m, int &tm,
                                            int &tn) {
  const int per_group = group_m * tiles_n;
  const int g = b / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gm = rows_left < group_m ? rows_left : group_m;
  const int in = b - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Map a linear workgroup id to a C tile (tm, tn).
//
// 1. XCD-aware remap.  Consecutive workgroup ids are dispatched round-robin
//    over the 8 XCDs, each with its own L2.  Renumber so that every XCD owns
//    one contiguous range of the tile order: XCD x holds ids x, x+8, x+16, ...
//    and gets the x-th slice.  The remap is a bijection for any count.
// 2. Grouped order.  Within the renumbered order, tiles run down a band of
//    `group_m` tile rows before moving one tile column right, so the
//    workgroups resident on one XCD at a time share A row panels and B column
//    panels in that XCD's L2.
//
// With a split-K launch the grid holds `splits` copies of the tile order, one
// per K chunk, after one another: the renumbered id gives the split (b / T for
// T tiles) and the tile within it, so an XCD's range covers tiles of the same
// K chunk, which share A and B panels.
//
// A launch over part of the order (tile_base, tiles) numbers its workgroups
// the same way over that part.
// `tiles`: tiles per split in this launch (they start at position tile_base
// of the grouped order); `local` receives the tile's index among them.
// Position of workgroup `bid` in an order where every XCD owns one
// contiguous range (step 1 below).
__device__ __forceinline__ int xcd_order(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int lid = bid / kXcds;
  const int q = nblocks / kXcds;
  const int r = nblocks % kXcds;
  return xcd * q + (xcd < r ? xcd : r) + lid;
}

__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int tiles, int tile_base, int &tm,
                                              int &tn, int &split, int &local) {
  int b = xcd_order(bid, nblocks);
  split = b / tiles;
  local = b - split * tiles;
  tile_coords(tile_base + local, tiles_m, tiles_n, group_m, tm, tn);
}

__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int &tm, int &tn, int &split) {
  int local;
  tile_of_block(bid, nblocks, tiles_m, tiles_n, group_m, tiles_m * tiles_n, 0, tm, tn, split,
                local);
}

// fp32 -> fp16 with round-to-nearest-even (v_cvt_f16_f32 under the default
// rounding mode; never the round-toward-zero packed form).  Overflow gives
// +-infinity.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}


// ---------------------------------------------------------------- pipeline helpers

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); counters not waited on are set to their maxima.
constexpr int wait_vmcnt(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);
constexpr int kWaitAll = 0;

// Buffer resource (V#) for raw byte-addressed loads from `base`: no stride,
// no swizzle, 32-bit data format, and the largest record count, so the
// hardware range check never clips (callers keep every access inside the
// matrix themselves).
typedef int BufRsrc __attribute__((ext_vector_type(4)));

__device__ __forceinline__ BufRsrc buffer_rsrc(const void *base) {
  const unsigned long long b = (unsigned long long)(uintptr_t)base;
  BufRsrc r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((b >> 32) & 0xffffu));
  r[2] = -1;
  r[3] = 0x00020000;
  return r;
}

// One 16-byte direct global->LDS load per lane: lane L loads the 16 bytes at
// byte offset `voff` from the resource's base and writes them to LDS bytes
// m0 + 16*L (m0 is wave-uniform).  Each lane sends a 32-bit offset rather
// than a 64-bit address, which measurably lowers the cost of the loads next
// to the MFMA work.  The load is written as inline assembly on purpose: the
// compiler's wait-count tracking then does not see it, and does not drain
// every outstanding direct load before each LDS read.  Completion is ensured
// explicitly instead: each wave waits on vmcnt for its own loads of a slot
// before the barrier that publishes the slot (the kernel's only other
// vector-memory loads come before the direct loads or after a full wait).
// The build checks that no compiler-generated instruction uses m0.
__device__ __forceinline__ void buffer_load16(uint32_t voff, BufRsrc rsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr)
               : "memory", "m0");
}

// Wait until at most `steps` K steps of this wave's direct loads are still in
// flight (LOADS load instructions per step; steps <= 0 waits for all of
// them), and for every LDS access.  More than three steps wait as for three.
template <int LOADS>
__device__ __forceinline__ void wait_direct(int steps) {
  static_assert(3 * LOADS <= 63, "vmcnt range");
  if (steps <= 0) __builtin_amdgcn_s_waitcnt(kWaitAll);
  else if (steps == 1) __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS) & kWaitLgkm0);
  else if (steps == 2) __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LOADS) & kWaitLgkm0);
  else __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * LOADS) & kWaitLgkm0);
}

// LDS byte address of a pointer into the kernel's shared array.
__device__ __forceinline__ uint32_t lds_address(const char *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Debug builds (DGEMM_LDS_POISON): fill a kernel's shared memory with
// 0x7FC07FC0, a NaN both as one binary32 value and as two binary16 values,
// before the kernel uses it, so that any read of LDS that the pipeline never
// wrote (a wrong offset, swizzle or staging row) turns the result into NaN
// and fails the parity tests.  Release builds compile this away.
__device__ __forceinline__ void lds_poison(void *lds, int bytes) {
#ifdef DGEMM_LDS_POISON
  uint32_t *w = static_cast<uint32_t *>(lds);
  for (int i = (int)threadIdx.x; i < bytes / 4; i += (int)blockDim.x) w[i] = 0x7FC07FC0u;
  __syncthreads();
#else
  (void)lds;
  (void)bytes;
#endif
}

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// Barrier that does not wait for outstanding loads; the asm statement keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K step kt covers [k0(kt), k0(kt) + BK); when K % BK != 0 the partial step
// comes first, then the full steps from k = 0.
struct KSteps {
  int nk, nfull, tail, bk;
  __device__ __forceinline__ int k0(int kt) const {
    return tail ? (kt == 0 ? nfull * bk : (kt - 1) * bk) : kt * bk;
  }
};

// Load width of an operand on the register-staged path, from GemmParams::vec_ab:
// 2 = 16-byte vectors, 1 = element pairs, 0 = single elements.
__device__ __forceinline__ int vec_width_a(int vec_ab) {
  return (vec_ab & 1) ? 2 : ((vec_ab & 4) ? 1 : 0);
}
__device__ __forceinline__ int vec_width_b(int vec_ab) {
  return (vec_ab & 2) ? 2 : ((vec_ab & 8) ? 1 : 0);
}

// vec_ab from the per-operand widths a plan chose (elements per access; the
// full vector width `vec` means 16 bytes).
inline int vec_bits(int vec_a, int vec_b, int vec) {
  return (vec_a == vec ? 1 : 0) | (vec_b == vec ? 2 : 0) | (vec_a == 2 ? 4 : 0) |
         (vec_b == 2 ? 8 : 0);
}

__device__ __forceinline__ KSteps make_steps(int K, int BK) {
  KSteps s;
  s.bk = BK;
  s.nfull = K / BK;
  s.tail = K % BK;
  s.nk = s.nfull + (s.tail ? 1 : 0);
  return s;
}

}  // namespace dgemm
