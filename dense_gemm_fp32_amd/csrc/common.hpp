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
};

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
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int &tm, int &tn) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int q = nblocks / kXcds;
  const int r = nblocks % kXcds;
  const int b = xcd * q + (xcd < r ? xcd : r) + local;
  const int per_group = group_m * tiles_n;
  const int g = b / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gm = rows_left < group_m ? rows_left : group_m;
  const int in = b - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
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

}  // namespace dgemm
