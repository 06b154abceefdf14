// pack.hip -- aligned copies of operands whose rows do not allow 16-byte loads.
//
// The GEMM kernels move A and B with 16-byte loads (straight from global
// memory into LDS) only when every row of the stored operand starts on a
// 16-byte boundary: ld a multiple of 4 floats or 8 halves and a 16-byte
// aligned base (the SGEMM summary's memory-layout section gives the
// condition for its 128-bit loads).  Otherwise they fall back to register-
// staged loads of pairs or single elements, which cost several times the load
// instructions per K step.  For a large enough call it is cheaper to copy such
// an operand once into a workspace whose rows are padded to a multiple of 16
// bytes (the pad holds zeros, which no kernel reads), and run the GEMM on the
// copy with the vector path: the copy reads and writes the operand once, at
// memory speed, where the staged loads pay on every K step of every tile that
// reads it.  The copy is bit-exact, so the products, their order and the
// result are those of the GEMM on the original operands under the same tile
// and split.
//
// The copy and the GEMM's own split-K workspace come from one workspace
// allocation; when it cannot be had, or the call is small (the rule below),
// the call runs on the original operands.
#include "common.hpp"
#include "internal.hpp"

namespace dgemm {

namespace {

constexpr int kPackThreads = 256;
constexpr unsigned kPackMaxBlocks = 2048;
constexpr size_t kPackAlign = 256;     // workspace sub-buffers start on 256-byte boundaries
// Largest workspace a call takes from the pool (the split-K cap in splitk.hip).
constexpr long long kPoolCallCap = 1LL << 30;

// One stored matrix to copy: rows x cols elements at src (row pitch ld_src
// elements) into dst (row pitch ld_dst elements, a multiple of 16 bytes);
// n = rows * ld_dst elements written.
struct PackJob {
  const void *src;
  void *dst;
  long long ld_src;
  unsigned ld_dst;
  int cols;
  long long n;
};

// Consecutive threads on consecutive elements of a row, so that every wave
// reads and writes one contiguous run of each matrix; elements past a row's
// last column are written as zeros.  Each thread takes kPackIlp elements a
// grid apart and issues all their loads before any store (a store could
// otherwise alias the next load and hold it back a full memory latency).
// Jobs j0 and j1 (A and B) share the launch: elements [0, j0.n) of the
// combined range are j0's.  WIDE: a job holds 2^32 elements or more (64-bit
// index arithmetic).
constexpr int kPackIlp = 8;

template <typename E, bool WIDE>
__device__ __forceinline__ const E *pack_source(const PackJob &j, long long u) {
  long long row;
  int col;
  if constexpr (WIDE) {
    row = u / j.ld_dst;
    col = (int)(u - row * j.ld_dst);
  } else {
    const unsigned uu = (unsigned)u;
    row = uu / j.ld_dst;
    col = (int)(uu - (unsigned)row * j.ld_dst);
  }
  return col < j.cols ? static_cast<const E *>(j.src) + row * j.ld_src + col : nullptr;
}

template <typename E, bool WIDE>
__global__ __launch_bounds__(kPackThreads) void pack_rows(PackJob j0, PackJob j1) {
  const long long total = j0.n + j1.n;
  const long long step = (long long)gridDim.x * kPackThreads;
  for (long long t0 = (long long)blockIdx.x * kPackThreads + threadIdx.x; t0 < total;
       t0 += step * kPackIlp) {
    E v[kPackIlp];
#pragma unroll
    for (int i = 0; i < kPackIlp; ++i) {
      const long long t = t0 + i * step;
      v[i] = E(0);
      if (t < total) {
        const bool second = t >= j0.n;
        const E *s = pack_source<E, WIDE>(second ? j1 : j0, second ? t - j0.n : t);
        if (s != nullptr) v[i] = *s;
      }
    }
#pragma unroll
    for (int i = 0; i < kPackIlp; ++i) {
      const long long t = t0 + i * step;
      if (t < total) {
        const bool second = t >= j0.n;
        static_cast<E *>(second ? j1.dst : j0.dst)[second ? t - j0.n : t] = v[i];
      }
    }
  }
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool rows_aligned(const void *p, int ld, int eb) {
  return (ld % (16 / eb)) == 0 && aligned_to(p, 16);
}

// Stored shape of A and B: A is M x K (K x M when transposed), B is K x N
// (N x K when transposed).
void stored_a(const Call &c, int *rows, int *cols) {
  *rows = c.ta ? c.K : c.M;
  *cols = c.ta ? c.M : c.K;
}
void stored_b(const Call &c, int *rows, int *cols) {
  *rows = c.tb ? c.N : c.K;
  *cols = c.tb ? c.K : c.N;
}

// Padded leading dimension (elements) of a copy of a matrix with `cols`
// columns, and the copy's bytes (whole 256-byte blocks).
int padded_ld(int cols, int eb) { return (int)round_up((size_t)cols, (size_t)(16 / eb)); }
size_t copy_bytes(int rows, int cols, int eb) {
  return round_up((size_t)rows * (size_t)padded_ld(cols, eb) * (size_t)eb, kPackAlign);
}

// Workspace a call may take: its fixed region, else its limit, else the
// pool's per-call cap.
long long ws_available(const Call &c) {
  if (c.ws_fixed != nullptr || c.ws_fixed_bytes > 0) return (long long)c.ws_fixed_bytes;
  if (c.ws_limit >= 0) return c.ws_limit < kPoolCallCap ? c.ws_limit : kPoolCallCap;
  return kPoolCallCap;
}

// The rule (fp32): copy when the call does at least kPackMinFlops flops, or
// at least kPackMinFlopsEvenN with N a multiple of 4 (then the copied call's
// last tile column still takes the direct loads; with a ragged N that column
// runs the masked staged path, and a grid of one round waits for it).
// Measured interleaved, copies forced on and off: the copy costs a launch of
// about 9 us for a few MB (latency-bound) plus the operands' bytes at memory
// speed; 2048^3 with every ld = 2049 +14-18%, 4096^3 +11-16%, 8192^3 +16%,
// 2000x2000x1000 +17-20%, 1000x1000x4000 +12-16%, 1536^3 +3-9%, the ragged
// 1000x3000x517 workload +21-29% (its copies take the four-wave 64x64 tile),
// 517x3000x1000 +4-12%, 1024^3 +5-7%, 1000^3 +3%; 1280^3 -4%; below the
// rule 768^3 -3%, 256^3 -11%, and 3000x517x1000 (N = 517) -20%.
// fp16 copies are made only when forced: the same measurements gave +10-23%
// on one box and -1 to -20% on another for the same shapes (2048^3, 4096^3,
// 8192^3 with ld = n + 1), so no size rule held.
constexpr double kPackMinFlops = 5.0e9;
constexpr double kPackMinFlopsEvenN = 1.5e9;

bool pack_by_size(const Call &c, int eb) {
  if (eb != 4) return false;
  const double flops = 2.0 * (double)c.M * (double)c.N * (double)c.K;
  return flops >= kPackMinFlops || (flops >= kPackMinFlopsEvenN && c.N % 4 == 0);
}

}  // namespace

PackChoice pack_choice(const Call &c, int eb, Plan (*plan)(const Call &)) {
  PackChoice pk;
  if (c.force_scalar || c.pack_mode == 1) return pk;
  const bool ua = !rows_aligned(c.A, c.lda, eb), ub = !rows_aligned(c.B, c.ldb, eb);
  if (!ua && !ub) return pk;
  if (c.pack_mode != 2 && !pack_by_size(c, eb)) return pk;
  int ra, ca, rb, cb;
  stored_a(c, &ra, &ca);
  stored_b(c, &rb, &cb);
  pk.a = ua;
  pk.b = ub;
  pk.lda = ua ? padded_ld(ca, eb) : c.lda;
  pk.ldb = ub ? padded_ld(cb, eb) : c.ldb;
  pk.a_bytes = ua ? copy_bytes(ra, ca, eb) : 0;
  pk.b_bytes = ub ? copy_bytes(rb, cb, eb) : 0;
  // The GEMM on the copies: planned with stand-in operand addresses that are
  // 16-byte aligned (planning looks only at their alignment).
  Call in = c;
  in.pack_mode = 1;
  if (ua) {
    in.A = reinterpret_cast<const void *>((uintptr_t)kPackAlign);
    in.lda = pk.lda;
  }
  if (ub) {
    in.B = reinterpret_cast<const void *>((uintptr_t)kPackAlign);
    in.ldb = pk.ldb;
  }
  pk.inner_ws = plan(in).ws_bytes;
  const size_t total = pk.a_bytes + pk.b_bytes + round_up(pk.inner_ws, kPackAlign);
  if ((long long)total > ws_available(c)) return PackChoice();
  pk.bytes = total;
  return pk;
}

Plan plan_packed(const Call &c, int eb, Plan (*plan)(const Call &)) {
  const PackChoice pk = pack_choice(c, eb, plan);
  if (!pk.a && !pk.b) return plan(c);
  Call in = c;
  in.pack_mode = 1;
  if (pk.a) {
    in.A = reinterpret_cast<const void *>((uintptr_t)kPackAlign);
    in.lda = pk.lda;
  }
  if (pk.b) {
    in.B = reinterpret_cast<const void *>((uintptr_t)kPackAlign);
    in.ldb = pk.ldb;
  }
  Plan pl = plan(in);
  pl.packed_a = pk.a;
  pl.packed_b = pk.b;
  pl.ws_bytes = pk.bytes;
  return pl;
}

hipError_t run_packed(const Call &c, int eb, Plan (*plan)(const Call &),
                      hipError_t (*launch)(const Call &)) {
  const PackChoice pk = pack_choice(c, eb, plan);
  if (!pk.a && !pk.b) return launch(c);
  void *ws = nullptr;
  if (workspace_alloc(c, pk.bytes, &ws) != hipSuccess) {
    Call plain = c;
    plain.pack_mode = 1;
    return launch(plain);
  }
  char *base = static_cast<char *>(ws);
  PackJob ja{}, jb{};
  Call in = c;
  in.pack_mode = 1;
  if (pk.a) {
    int rows, cols;
    stored_a(c, &rows, &cols);
    ja = PackJob{c.A, base, c.lda, (unsigned)pk.lda, cols, (long long)rows * pk.lda};
    in.A = base;
    in.lda = pk.lda;
  }
  if (pk.b) {
    int rows, cols;
    stored_b(c, &rows, &cols);
    char *dst = base + pk.a_bytes;
    jb = PackJob{c.B, dst, c.ldb, (unsigned)pk.ldb, cols, (long long)rows * pk.ldb};
    in.B = dst;
    in.ldb = pk.ldb;
  }
  // The GEMM's own workspace (split K) is the rest of the allocation.
  in.ws_fixed = base + pk.a_bytes + pk.b_bytes;
  in.ws_fixed_bytes = pk.bytes - pk.a_bytes - pk.b_bytes;
  const long long total = ja.n + jb.n;
  long long blocks = (total + kPackThreads * kPackIlp - 1) / (kPackThreads * kPackIlp);
  if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
  if (blocks < 1) blocks = 1;
  const bool wide = ja.n >= (1LL << 32) || jb.n >= (1LL << 32);
  const dim3 g((unsigned)blocks), b(kPackThreads);
  if (eb == 4) {
    if (wide) hipLaunchKernelGGL((pack_rows<uint32_t, true>), g, b, 0, c.stream, ja, jb);
    else hipLaunchKernelGGL((pack_rows<uint32_t, false>), g, b, 0, c.stream, ja, jb);
  } else {
    if (wide) hipLaunchKernelGGL((pack_rows<uint16_t, true>), g, b, 0, c.stream, ja, jb);
    else hipLaunchKernelGGL((pack_rows<uint16_t, false>), g, b, 0, c.stream, ja, jb);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch(in);
  const hipError_t f = workspace_free(c, ws);
  return e != hipSuccess ? e : f;
}

}  // namespace dgemm
