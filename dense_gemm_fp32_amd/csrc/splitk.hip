// splitk.hip -- the second half of a split-K GEMM and its workspace.
//
// When a problem's tile grid leaves CUs idle, the GEMM kernels can divide K
// into S chunks (the independent, tile-sized units of the SGEMM summary's
// tiling section, multiplied by S along K) and write each chunk's raw fp32
// sums to its own slab of a workspace.  splitk_reduce then forms, for every
// element,
//
//     C := alpha * (W_0 + W_1 + ... + W_{S-1}) + beta * C
//
// summing the slabs in that fixed order in fp32, so the result is the same
// bits on every call with the same shape and split count (no atomics, no
// arrival-order dependence).  alpha*sum + beta*C is formed in fp32 and, for an
// fp16 C, rounded once to half with round-to-nearest-even, exactly as the
// single-pass epilogues do.  C is read only when beta != 0.
//
// The workspace comes from a memory pool the library owns, one per device,
// with stream-ordered allocation on the call's stream: it is taken before
// the GEMM pass and given back after the reduction, in stream order, so
// concurrent calls on different streams never share it and nothing is
// synchronised.  Freed blocks stay in the pool for later calls up to a release
// threshold (kPoolKeep), beyond which the runtime returns the memory at the
// next synchronisation; every request is made at the largest size used so far
// (see workspace_alloc).  A caller may cap the workspace of a call
// (gemm_set_workspace_limit); a call that cannot get its workspace runs
// unsplit.
//
// The entry point that allocates nothing takes its workspace from `scratch`,
// a file-scope device array of fixed size, instead of the pool.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

namespace {

constexpr int kMaxDevices = 64;
// Freed workspace the pool keeps for later calls; memory beyond it goes back
// to the runtime at the next synchronisation.
constexpr uint64_t kPoolKeep = (uint64_t)256 << 20;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices];
bool g_pool_made[kMaxDevices];
size_t g_high_water[kMaxDevices];   // largest workspace requested so far, per device

hipError_t pool_for(int dev, hipMemPool_t *out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool_made[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipError_t e = hipMemPoolCreate(&g_pool[dev], &props);
    if (e != hipSuccess) return e;
    uint64_t keep = kPoolKeep;
    e = hipMemPoolSetAttribute(g_pool[dev], hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    g_pool_made[dev] = true;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

// The no-allocation entry point's workspace: one copy per device, alive until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device memory: its device address comes from hipGetSymbolAddress,
// looked up once per device (with that device current) and kept.
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

constexpr int kReduceThreads = 256;
constexpr unsigned kReduceMaxBlocks = 8192;

template <bool HALF_OUT, bool VEC_C, bool READ_C>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce(const float *__restrict__ W,
                                                                long long stride, int ldw, int S,
                                                                int M, int N, float alpha,
                                                                float beta, void *Cv, int ldc) {
  const long long groups = (long long)((N + 3) / 4);   // 4 adjacent columns per thread
  const long long total = (long long)M * groups;
  for (long long t = (long long)blockIdx.x * kReduceThreads + threadIdx.x; t < total;
       t += (long long)gridDim.x * kReduceThreads) {
    const int i = (int)(t / groups);
    const int j = 4 * (int)(t - (long long)i * groups);
    // ldw is a multiple of 4 and covers N, so the 16-byte loads stay inside
    // the slab; lanes past N carry values that are never stored.
    const float *w = W + (size_t)i * (size_t)ldw + j;
    f32x4 sum = *reinterpret_cast<const f32x4 *>(w);
    for (int s = 1; s < S; ++s) sum += *reinterpret_cast<const f32x4 *>(w + (size_t)s * stride);
    if constexpr (HALF_OUT) {
      uint16_t *c = static_cast<uint16_t *>(Cv) + (size_t)i * (size_t)ldc + j;
      if (VEC_C && j + 3 < N) {
        u32x2 cw = u32x2{0u, 0u};
        if (READ_C) cw = *reinterpret_cast<const u32x2 *>(c);
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o = alpha * sum[e];
          if (READ_C) {
            const uint16_t ce = (uint16_t)((e < 2 ? cw[0] : cw[1]) >> (16 * (e & 1)));
            o = __builtin_fmaf(beta, f16_bits_to_f32(ce), o);
          }
          h[e] = f32_to_f16_bits(o);
        }
        u32x2 ow;
        ow[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        ow[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<u32x2 *>(c) = ow;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j + e >= N) continue;
          float o = alpha * sum[e];
          if (READ_C) o = __builtin_fmaf(beta, f16_bits_to_f32(c[e]), o);
          c[e] = f32_to_f16_bits(o);
        }
      }
    } else {
      float *c = static_cast<float *>(Cv) + (size_t)i * (size_t)ldc + j;
      if (VEC_C && j + 3 < N) {
        f32x4 o;
        if (READ_C) {
          const f32x4 cv = *reinterpret_cast<const f32x4 *>(c);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(beta, cv[e], alpha * sum[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = alpha * sum[e];
        }
        *reinterpret_cast<f32x4 *>(c) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j + e >= N) continue;
          float o = alpha * sum[e];
          if (READ_C) o = __builtin_fmaf(beta, c[e], o);
          c[e] = o;
        }
      }
    }
  }
}

template <bool HALF_OUT, bool VEC_C>
hipError_t reduce_launch(const SplitReduce &r, hipStream_t s) {
  const long long total = (long long)r.M * (long long)((r.N + 3) / 4);
  long long blocks = (total + kReduceThreads - 1) / kReduceThreads;
  if (blocks > kReduceMaxBlocks) blocks = kReduceMaxBlocks;
  if (blocks < 1) blocks = 1;
  if (r.beta != 0.0f)
    hipLaunchKernelGGL((splitk_reduce<HALF_OUT, VEC_C, true>), dim3((unsigned)blocks),
                       dim3(kReduceThreads), 0, s, r.W, r.stride, r.ldw, r.S, r.M, r.N, r.alpha,
                       r.beta, r.C, r.ldc);
  else
    hipLaunchKernelGGL((splitk_reduce<HALF_OUT, VEC_C, false>), dim3((unsigned)blocks),
                       dim3(kReduceThreads), 0, s, r.W, r.stride, r.ldw, r.S, r.M, r.N, r.alpha,
                       r.beta, r.C, r.ldc);
  return hipGetLastError();
}

// One thread per 4 adjacent columns of a tile row: sum the S dense blocks in
// order s = 0..S-1, then alpha*sum + beta*C on the elements inside the
// matrix.  Blocks are BM x BN with BN a multiple of 4, so the 16-byte loads
// stay inside each block.
template <bool VEC_C, bool READ_C>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_tiles(TileReduce r) {
  const int groups = r.BN / 4;
  const long long per_tile = (long long)r.BM * groups;
  const long long total = (long long)r.tiles * per_tile;
  const size_t block = (size_t)r.BM * (size_t)r.BN;
  for (long long t = (long long)blockIdx.x * kReduceThreads + threadIdx.x; t < total;
       t += (long long)gridDim.x * kReduceThreads) {
    const int lt = (int)(t / per_tile);
    const int rem = (int)(t - (long long)lt * per_tile);
    const int i = rem / groups;
    const int j = 4 * (rem - i * groups);
    int tm, tn;
    tile_coords(r.tile_base + lt, r.tiles_m, r.tiles_n, r.group_m, tm, tn);
    const int row = tm * r.BM + i, col = tn * r.BN + j;
    if (row >= r.M || col >= r.N) continue;
    const float *w = r.W + (size_t)lt * block + (size_t)i * r.BN + j;
    f32x4 sum = *reinterpret_cast<const f32x4 *>(w);
    for (int s = 1; s < r.S; ++s)
      sum += *reinterpret_cast<const f32x4 *>(w + (size_t)s * (size_t)r.tiles * block);
    float *c = r.C + (size_t)row * (size_t)r.ldc + col;
    if (VEC_C && col + 3 < r.N) {
      f32x4 o;
      if (READ_C) {
        const f32x4 cv = *reinterpret_cast<const f32x4 *>(c);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(r.beta, cv[e], r.alpha * sum[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = r.alpha * sum[e];
      }
      *reinterpret_cast<f32x4 *>(c) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= r.N) continue;
        float o = r.alpha * sum[e];
        if (READ_C) o = __builtin_fmaf(r.beta, c[e], o);
        c[e] = o;
      }
    }
  }
}

// One thread per 4 adjacent columns of a tile row, over every tile; tiles
// that one workgroup covered whole were written by the GEMM and are skipped.
template <bool VEC_C, bool READ_C>
__global__ __launch_bounds__(kReduceThreads) void streamk_fixup(StreamKFixup f) {
  const int groups = f.BN / 4;
  const long long per_tile = (long long)f.BM * groups;
  const long long total = (long long)(f.tiles - f.tile_base) * per_tile;
  const size_t block = (size_t)f.BM * (size_t)f.BN;
  for (long long t = (long long)blockIdx.x * kReduceThreads + threadIdx.x; t < total;
       t += (long long)gridDim.x * kReduceThreads) {
    const int local = (int)(t / per_tile);
    const long long first_it = (long long)local * f.steps;
    const long long g0 = first_it / f.iters;
    const long long g1 = (first_it + f.steps - 1) / f.iters;
    if (g0 == g1) continue;
    const int rem = (int)(t - (long long)local * per_tile);
    const int i = rem / groups;
    const int j = 4 * (rem - i * groups);
    int tm, tn;
    tile_coords(f.tile_base + local, f.tiles_m, f.tiles_n, f.group_m, tm, tn);
    const int row = tm * f.BM + i, col = tn * f.BN + j;
    if (row >= f.M || col >= f.N) continue;
    // workgroup g holds this tile in its last segment if the tile starts
    // after g's run does, else in its first
    f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (long long g = g0; g <= g1; ++g) {
      const long long slot = 2 * g + (first_it > g * f.iters ? 1 : 0);
      sum += *reinterpret_cast<const f32x4 *>(f.W + (size_t)slot * block + (size_t)i * f.BN + j);
    }
    float *c = f.C + (size_t)row * (size_t)f.ldc + col;
    if (VEC_C && col + 3 < f.N) {
      f32x4 o;
      if (READ_C) {
        const f32x4 cv = *reinterpret_cast<const f32x4 *>(c);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(f.beta, cv[e], f.alpha * sum[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f.alpha * sum[e];
      }
      *reinterpret_cast<f32x4 *>(c) = o;
    } else {
      float cv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cv[e] = (READ_C && col + e < f.N) ? c[e] : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= f.N) continue;
        float o = f.alpha * sum[e];
        if (READ_C) o = __builtin_fmaf(f.beta, cv[e], o);
        c[e] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_streamk_fixup(const StreamKFixup &f, hipStream_t s) {
  const long long total = (long long)(f.tiles - f.tile_base) * f.BM * (f.BN / 4);
  long long blocks = (total + kReduceThreads - 1) / kReduceThreads;
  if (blocks > kReduceMaxBlocks) blocks = kReduceMaxBlocks;
  if (blocks < 1) blocks = 1;
  const bool vec = !f.force_scalar && (f.ldc % 4) == 0 && aligned_to(f.C, 16);
  const dim3 g((unsigned)blocks), b(kReduceThreads);
  if (f.beta != 0.0f) {
    if (vec) hipLaunchKernelGGL((streamk_fixup<true, true>), g, b, 0, s, f);
    else hipLaunchKernelGGL((streamk_fixup<false, true>), g, b, 0, s, f);
  } else {
    if (vec) hipLaunchKernelGGL((streamk_fixup<true, false>), g, b, 0, s, f);
    else hipLaunchKernelGGL((streamk_fixup<false, false>), g, b, 0, s, f);
  }
  return hipGetLastError();
}

hipError_t launch_tile_reduce(const TileReduce &r, hipStream_t s) {
  const long long total = (long long)r.tiles * r.BM * (r.BN / 4);
  long long blocks = (total + kReduceThreads - 1) / kReduceThreads;
  if (blocks > kReduceMaxBlocks) blocks = kReduceMaxBlocks;
  if (blocks < 1) blocks = 1;
  const bool vec = !r.force_scalar && (r.ldc % 4) == 0 && aligned_to(r.C, 16);
  const dim3 g((unsigned)blocks), b(kReduceThreads);
  if (r.beta != 0.0f) {
    if (vec) hipLaunchKernelGGL((splitk_reduce_tiles<true, true>), g, b, 0, s, r);
    else hipLaunchKernelGGL((splitk_reduce_tiles<false, true>), g, b, 0, s, r);
  } else {
    if (vec) hipLaunchKernelGGL((splitk_reduce_tiles<true, false>), g, b, 0, s, r);
    else hipLaunchKernelGGL((splitk_reduce_tiles<false, false>), g, b, 0, s, r);
  }
  return hipGetLastError();
}

// Largest workspace a split-K call takes; beyond it the call runs unsplit.
constexpr long long kWorkspaceCap = 1LL << 30;

int clamp_splits(const Call &c, int want, int bk, long long tiles, int *k_chunk,
                 long long ws_elems_per_split) {
  *k_chunk = 0;
  int S = c.split_mode == 1 ? 1 : (c.split_mode >= 2 ? c.split_mode : want);
  const int steps = (c.K + bk - 1) / bk;
  if (S > steps) S = steps;
  if (S < 2) return 1;
  const int kc = ((c.K + S - 1) / S + bk - 1) / bk * bk;   // whole K steps per chunk
  S = (c.K + kc - 1) / kc;                                   // chunks actually needed
  if (S < 2) return 1;
  if (tiles * (long long)S > 0x7fffffffLL) return 1;
  const long long ldw = ((long long)c.N + 3) / 4 * 4;
  const long long per = ws_elems_per_split > 0 ? ws_elems_per_split : (long long)c.M * ldw;
  if ((long long)S * per * (long long)sizeof(float) > kWorkspaceCap) return 1;
  *k_chunk = kc;
  return S;
}

int stream_device(hipStream_t s) {
  int dev = -1;
  if (s != nullptr && hipStreamGetDevice(s, &dev) == hipSuccess) return dev;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return dev;
}

hipError_t scratch_region(int dev, void **ptr) {
  *ptr = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Pool requests ask for the largest size requested so far on the device (in
// 2 MiB steps), so a freed block always fits the next request: measured, a
// request larger than the blocks the pool holds costs ~30 us more than one it
// can serve from a freed block, and the pool does not reuse a block across
// different sizes.  That size rises only up to what the pool keeps: a block
// larger than kPoolKeep goes back to the runtime at the next
// synchronisation, so raising every later request to it would make each
// such request a fresh allocation of that size.  Larger requests are made at
// their own size.  A call with a fixed region uses it when it is large
// enough and never touches the pool.
hipError_t workspace_alloc(const Call &c, size_t bytes, void **ptr) {
  *ptr = nullptr;
  if (c.ws_fixed != nullptr) {
    if (bytes > c.ws_fixed_bytes) return hipErrorOutOfMemory;
    *ptr = c.ws_fixed;
    return hipSuccess;
  }
  if (c.ws_limit >= 0 && (long long)bytes > c.ws_limit) return hipErrorOutOfMemory;
  const int dev = stream_device(c.stream);
  hipMemPool_t pool;
  hipError_t e = pool_for(dev, &pool);
  if (e != hipSuccess) return e;
  constexpr size_t kStep = 2u << 20;
  bytes = (bytes + kStep - 1) / kStep * kStep;
  {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (bytes <= kPoolKeep) {
      if (bytes > g_high_water[dev]) g_high_water[dev] = bytes;
      bytes = g_high_water[dev];
    }
  }
  e = hipMallocFromPoolAsync(ptr, bytes, pool, c.stream);
  if (e != hipSuccess) {
    *ptr = nullptr;
    (void)hipGetLastError();   // a failed allocation is not the caller's error
  }
  return e;
}

hipError_t workspace_free(const Call &c, void *ptr) {
  if (ptr == nullptr || c.ws_fixed != nullptr) return hipSuccess;
  return hipFreeAsync(ptr, c.stream);
}

hipError_t launch_splitk_reduce(const SplitReduce &r, hipStream_t s) {
  const uintptr_t need = r.half_out ? 8 : 16;
  const bool vec = !r.force_scalar && (r.ldc % 4) == 0 && aligned_to(r.C, need);
  if (r.half_out) return vec ? reduce_launch<true, true>(r, s) : reduce_launch<true, false>(r, s);
  return vec ? reduce_launch<false, true>(r, s) : reduce_launch<false, false>(r, s);
}

}  // namespace dgemm
