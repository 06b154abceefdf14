// scale.hip -- the degenerate GEMM paths: when alpha == 0 or K == 0 the
// product term vanishes and C := beta * C (beta == 0 writes zeros without
// reading C).  Memory-bound elementwise pass; one thread per element of a
// row segment, rows spread over the grid's y dimension.
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

constexpr int kScaleThreads = 256;
constexpr int kScaleMaxRowsPerGrid = 65535;

template <bool ZERO>
__global__ __launch_bounds__(kScaleThreads) void scale_f32(int M, int N, float beta, float *C,
                                                           int ldc) {
  const int j = blockIdx.x * kScaleThreads + threadIdx.x;
  if (j >= N) return;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    float *p = C + (size_t)i * (size_t)ldc + j;
    *p = ZERO ? 0.0f : beta * *p;
  }
}

template <bool ZERO>
__global__ __launch_bounds__(kScaleThreads) void scale_f16(int M, int N, float beta, uint16_t *C,
                                                           int ldc) {
  const int j = blockIdx.x * kScaleThreads + threadIdx.x;
  if (j >= N) return;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    uint16_t *p = C + (size_t)i * (size_t)ldc + j;
    *p = ZERO ? (uint16_t)0 : f32_to_f16_bits(beta * f16_bits_to_f32(*p));
  }
}

static dim3 scale_grid(int M, int N) {
  const unsigned gx = (unsigned)((N + kScaleThreads - 1) / kScaleThreads);
  const unsigned gy = (unsigned)(M < kScaleMaxRowsPerGrid ? M : kScaleMaxRowsPerGrid);
  return dim3(gx, gy);
}

hipError_t launch_scale_f32(int M, int N, float beta, float *C, int ldc, hipStream_t s) {
  if (beta == 0.0f)
    hipLaunchKernelGGL(scale_f32<true>, scale_grid(M, N), dim3(kScaleThreads), 0, s, M, N, beta, C,
                       ldc);
  else
    hipLaunchKernelGGL(scale_f32<false>, scale_grid(M, N), dim3(kScaleThreads), 0, s, M, N, beta, C,
                       ldc);
  return hipGetLastError();
}

hipError_t launch_scale_f16(int M, int N, float beta, uint16_t *C, int ldc, hipStream_t s) {
  if (beta == 0.0f)
    hipLaunchKernelGGL(scale_f16<true>, scale_grid(M, N), dim3(kScaleThreads), 0, s, M, N, beta, C,
                       ldc);
  else
    hipLaunchKernelGGL(scale_f16<false>, scale_grid(M, N), dim3(kScaleThreads), 0, s, M, N, beta, C,
                       ldc);
  return hipGetLastError();
}

}  // namespace dgemm
