// internal.hpp -- host-side interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgemm {

// One validated GEMM call, after quick returns have been taken: M, N, K > 0
// and alpha != 0.
struct Call {
  int M, N, K;
  float alpha, beta;
  const void *A;
  int lda;
  const void *B;
  int ldb;
  void *C;
  int ldc;
  bool out32;            // fp16 inputs: C and the result are fp32 (else fp16)
  bool ta, tb;           // A stored transposed (K x M, lda >= M) / B (N x K, ldb >= K)
  bool force_scalar;     // diagnostic: element-wise loads/stores everywhere
  int split_mode;        // 0 = split K by size, 1 = never, >= 2 = that many splits (diagnostic)
  // Set by the launcher for the partial pass of a split-K call (else 1, 0, 0).
  int splits;
  int k_chunk;
  long long split_stride;
  // Set by the launcher for a launch over part of the tile order (else 0, 0,
  // false): tiles [tile_base, tile_base + tile_count) of the grouped order;
  // c_tiles: the split-K pass writes dense per-(split, tile) blocks.
  int tile_base, tile_count;
  bool c_tiles;
  int tail_mode;         // 0 = split the last round's tiles by size, 1 = never, >= 2 = that many (diagnostic)
  int tile_config;       // diagnostic: 0 = by size, 1/2/3/4 = large/medium/small/tiny,
                         // 5 = medium with the loads of a step issued together,
                         // 6 = fp32 256x256 (fp16: its large tile),
                         // 7 = fp32 64x64 with four waves (fp16: its small tile),
                         // 8 = fp32 128x64 with four waves (fp16: its medium tile),
                         // 9 = fp32 64x64 four waves, 64-k steps (fp16: its small tile),
                         // 10 = fp32 32x32 one wave, 64-k steps (fp16: its small tile)
  // Split-K workspace source: the library's per-device pool (ws_fixed ==
  // nullptr), requests above ws_limit bytes failing (-1: no limit), or a
  // fixed device region of ws_fixed_bytes bytes that is never allocated or
  // freed (the entry point that allocates nothing).
  long long ws_limit;
  void *ws_fixed;
  size_t ws_fixed_bytes;
  // Copies of A and B with 16-byte rows (pack.hip): 0 = when an operand's rows
  // do not allow 16-byte loads and the call is large enough, 1 = never,
  // 2 = whenever an operand's rows do not allow them (diagnostic).
  int pack_mode;
  // Stream-K (fp32): 0 = by size, 1 = never, 2..6 = in that mode (see
  // streamk_geometry) whenever the four-wave 64x64 tile or a forced tile
  // configuration (1, 5, 6, 7) is taken.
  int streamk_mode;
  hipStream_t stream;
};

// Chosen kernel variant (for launching and for gemm_describe).
struct Plan {
  const char *name;      // tile configuration, e.g. "f32 mfma32x32x2 128x128x32 w2x2"
  int bm, bn, bk;
  int threads;
  int vec_a, vec_b, vec_c;   // elements per global access (1 = scalar)
  long long blocks;          // tiles
  int splits;                // K chunks (1 = no split)
  int tail;                  // K chunks of the last round's tiles (1 = none)
  size_t ws_bytes;           // workspace the call takes: copies of A and B, split K (0 = none)
  bool packed_a = false;     // the GEMM runs on a 16-byte-row copy of A ...
  bool packed_b = false;     // ... of B
  bool streamk = false;      // Stream-K over `blocks` workgroups, then a fix-up pass ...
  long long sk_whole = 0;    // ... the first sk_whole of them computing whole tiles
};

// The reduction pass of a split-K run of tiles: for each of `tiles` tiles
// (positions tile_base.. of the grouped order over a tiles_m x tiles_n grid
// of BM x BN tiles), C := alpha * sum_s W[s][tile] + beta * C on the part of
// the tile inside the M x N matrix; W[s][tile] is a dense BM x BN fp32 block
// at W + (s*tiles + tile)*BM*BN.  fp32 C.
struct TileReduce {
  const float *W;
  int S, tiles, tile_base;
  int BM, BN, tiles_m, tiles_n, group_m;
  int M, N;
  float alpha, beta;
  float *C;
  int ldc;
  bool force_scalar;
};
hipError_t launch_tile_reduce(const TileReduce &r, hipStream_t s);

// The fix-up pass of a Stream-K launch: tiles tile_base .. tiles-1 of
// `steps` K steps each, dealt out in runs of `iters` steps per Stream-K
// workgroup; for every tile that more than one workgroup covered, C :=
// alpha * (sum of its workgroups' partial blocks, in workgroup order) +
// beta * C on the part of the tile inside the matrix.  Stream-K workgroup
// g's partial blocks are W[2g] (its first segment) and W[2g + 1] (its last),
// dense BM x BN fp32 each.  fp32 C.
struct StreamKFixup {
  const float *W;
  int tiles, tile_base, steps;
  long long iters;
  int BM, BN, tiles_m, tiles_n, group_m;
  int M, N;
  float alpha, beta;
  float *C;
  int ldc;
  bool force_scalar;
};
hipError_t launch_streamk_fixup(const StreamKFixup &f, hipStream_t s);

// The reduction pass of a split-K call: C := alpha * sum_s W_s + beta * C over
// an M x N matrix, the S slabs of W (fp32, row pitch ldw, `stride` floats
// apart) summed in order s = 0..S-1.
struct SplitReduce {
  const float *W;
  long long stride;
  int ldw, S, M, N;
  float alpha, beta;
  void *C;
  int ldc;
  bool half_out;       // C is fp16 (else fp32)
  bool force_scalar;
};

// Split-K workspace of `bytes` bytes for call c, ordered on c.stream: from
// c's fixed region when it has one (no allocation; fails if too small), else
// from the library's per-device memory pool (fails above c.ws_limit).  A
// launcher that cannot get its workspace runs the call unsplit.
hipError_t workspace_alloc(const Call &c, size_t bytes, void **ptr);
hipError_t workspace_free(const Call &c, void *ptr);

// Bytes of a whole split-K workspace (S slabs of M x ceil(N/4)*4 floats) and
// of a last-round split (S dense BM x BN fp32 blocks per leftover tile).
inline size_t split_ws_bytes(int S, int M, int N) {
  return (size_t)S * (size_t)M * (size_t)((N + 3) / 4 * 4) * sizeof(float);
}
inline size_t tail_ws_bytes(int S, int tiles, int BM, int BN) {
  return (size_t)S * (size_t)tiles * (size_t)BM * (size_t)BN * sizeof(float);
}

// The fixed scratch region of the entry point that allocates nothing: a
// file-scope device array of kScratchBytes bytes, its address on device
// `dev` looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_region(int dev, void **ptr);
// Device a stream belongs to (NULL stream: the current device); -1 on error.
int stream_device(hipStream_t s);
hipError_t launch_splitk_reduce(const SplitReduce &r, hipStream_t s);

// Split count for a problem with `tiles` tiles of K step `bk`, given the
// call's split mode and the heuristic's choice `want` (1 = no split): clamped
// so every split has at least one K step, the grid stays within range and the
// workspace under its cap (ws_elems_per_split floats per split; 0: an M x N
// slab).  Also returns the chunk length.
int clamp_splits(const Call &c, int want, int bk, long long tiles, int *k_chunk,
                 long long ws_elems_per_split = 0);

// Copies of A and B whose rows allow 16-byte loads (pack.hip).  pack_choice:
// which operands of call c (elements of eb bytes: 4 or 2) are copied and the
// workspace that takes, including the split-K workspace of the GEMM on the
// copies (planned by `plan`); nothing is copied when both operands already
// allow 16-byte loads, under the test switches, for small calls, or when the
// total exceeds the workspace the call may take.  plan_packed / run_packed:
// the plan and the launch of call c with those copies (the copy kernel, then
// `launch` on the copies, on c's stream, from one workspace allocation; the
// call runs on the original operands when that allocation fails).
struct PackChoice {
  bool a = false, b = false;
  int lda = 0, ldb = 0;            // leading dimensions of the copies
  size_t a_bytes = 0, b_bytes = 0;
  size_t inner_ws = 0;             // split-K workspace of the GEMM on the copies
  size_t bytes = 0;                // the whole workspace
};
PackChoice pack_choice(const Call &c, int eb, Plan (*plan)(const Call &));

// Workspace a call may take: its fixed region, else its limit, else the
// pool's per-call cap.
long long ws_available(const Call &c);
Plan plan_packed(const Call &c, int eb, Plan (*plan)(const Call &));
hipError_t run_packed(const Call &c, int eb, Plan (*plan)(const Call &),
                      hipError_t (*launch)(const Call &));

Plan plan_f32(const Call &c);
Plan plan_f16(const Call &c);
hipError_t launch_f32(const Call &c);
// fp32 on the vector ALUs (the SIMT register-blocked design; ablation).
hipError_t launch_f32_valu(const Call &c);

// Matrix-core ceiling probe (probe.hip): buffer sizes it needs, its flop
// count per launch, and the launch (dtype 0 = fp32, 1 = fp16).
size_t probe_operand_bytes();
size_t probe_out_bytes();
double probe_flops(int dtype, int iters);
hipError_t launch_probe(int dtype, int iters, const void *operands, float *out, hipStream_t s);
hipError_t launch_f16(const Call &c);

// C := beta * C over an M x N matrix (beta == 0 writes zeros without reading).
hipError_t launch_scale_f32(int M, int N, float beta, float *C, int ldc, hipStream_t s);
hipError_t launch_scale_f16(int M, int N, float beta, uint16_t *C, int ldc, hipStream_t s);

inline bool aligned_to(const void *p, uintptr_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

}  // namespace dgemm
