// probe.hip -- matrix-core ceiling probe (a measurement aid, not a GEMM).
//
// The GEMM kernels' throughput is bounded by the MFMA rate at whatever clock
// the part sustains under their load.  This kernel measures that bound on the
// same hardware with no memory traffic at all: every wave loads its operand
// registers once, then issues `iters` rounds of independent MFMAs (the
// instruction and blocks of the large GEMM tiles' 128 x 64 wave tiles: fp16
// v_mfma_f32_16x16x32_f16 on 8 x 4 blocks of 16x16, fp32
// v_mfma_f32_32x32x2_f32 on 4 x 2 blocks of 32x32), and finally writes the sum
// of its accumulators so that no MFMA is dead.  The operand values come from the caller's buffer, so the
// probe switches the same bits as a GEMM on data of that distribution (the
// matrix cores' power, and with it the sustained clock, depends on them).
//
// Grid: kProbeBlocks workgroups of 512 threads (two per CU on 256 CUs, eight
// waves each).  Flops per launch = waves x iters x 2*128*64*k per round
// (k = 32 for fp16, 2 for fp32).
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 2 * kCUs;
constexpr int kOperandElems = 4096;   // operand vectors (16 B for fp16, 4 B for fp32) in the buffer

template <bool HALF>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe(const void *src, float *out, int iters) {
  const int t = blockIdx.x * kProbeThreads + threadIdx.x;
  if constexpr (HALF) {
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    const f16x8 *s = static_cast<const f16x8 *>(src);
    f16x8 a[8], b[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = s[(t * 7 + i) % kOperandElems];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = s[(t * 13 + 5 + j) % kOperandElems];
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += acc[i][j][r];
    out[t] = sum;
  } else {
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const float *s = static_cast<const float *>(src);
    float a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = s[(t * 7 + i) % kOperandElems];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = s[(t * 13 + 5 + j) % kOperandElems];
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
    out[t] = sum;
  }
}

}  // namespace

size_t probe_operand_bytes() { return (size_t)kOperandElems * 16; }
size_t probe_out_bytes() { return (size_t)kProbeBlocks * kProbeThreads * sizeof(float); }

double probe_flops(int dtype, int iters) {
  const double waves = (double)kProbeBlocks * kProbeThreads / kWave;
  // one round: the 128 x 64 wave tile over 32 k (fp16) or 2 k (fp32)
  const double per_round = 2.0 * 128 * 64 * (dtype == 1 ? 32 : 2);
  return waves * iters * per_round;
}

hipError_t launch_probe(int dtype, int iters, const void *operands, float *out, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(mfma_probe<true>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, operands,
                       out, iters);
  else
    hipLaunchKernelGGL(mfma_probe<false>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, operands,
                       out, iters);
  return hipGetLastError();
}

}  // namespace dgemm
