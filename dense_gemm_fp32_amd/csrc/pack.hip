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
constexpr unsigned kPackMaxBlocks = 8192;
constexpr size_t kPackAlign = 256;     // workspace sub-buffers start on 256-byte boundaries
// Largest workspace a call takes from the pool (the split-K cap in splitk.hip).
constexpr long long kPoolCallCap = 1LL << 30;

// One stored matrix to copy: `rows` rows of row_bytes bytes (cols elements)
// at src, row pitch src_pitch bytes, into dst, whose rows are cpr 16-byte
// chunks; n = rows * cpr chunks written.
struct PackJob {
  const char *src;
  char *dst;
  long long src_pitch;
  long long row_bytes;
  unsigned cpr;
  long long n;
};

// One 16-byte chunk of a destination row per thread.  The chunk's source
// bytes start anywhere on an element boundary, so they are read as the one or
// two aligned 16-byte granules that hold them and shifted into place: two
// 16-byte loads instead of four (fp32) or eight (fp16) element loads, and one
// 16-byte store.  The first granule holds the chunk's first byte; the second
// is read only when the chunk needs bytes from it that lie inside the row.
// A granule that holds any byte of the matrix lies in the same page as that
// byte, so no read can touch a page the matrix does not; bytes read from
// outside the row are never used.  Bytes past the row's last column are
// written as zeros.  Consecutive threads take consecutive chunks, so every
// wave reads and writes contiguous runs.  Jobs j0 and j1 (A and B) share the
// launch: chunks [0, j0.n) of the combined range are j0's.  WIDE: a job holds
// 2^32 chunks or more (64-bit index arithmetic).
template <bool WIDE>
__global__ __launch_bounds__(kPackThreads) void pack_rows(PackJob j0, PackJob j1) {
  const long long total = j0.n + j1.n;
  for (long long t = (long long)blockIdx.x * kPackThreads + threadIdx.x; t < total;
       t += (long long)gridDim.x * kPackThreads) {
    // the job's fields by value (a reference to one of the two arguments
    // would put them in scratch memory)
    const bool second = t >= j0.n;
    const long long u = second ? t - j0.n : t;
    const char *src = second ? j1.src : j0.src;
    char *dst = second ? j1.dst : j0.dst;
    const long long pitch = second ? j1.src_pitch : j0.src_pitch;
    const long long row_bytes = second ? j1.row_bytes : j0.row_bytes;
    const unsigned cpr = second ? j1.cpr : j0.cpr;
    long long row, chunk;
    if constexpr (WIDE) {
      row = u / cpr;
      chunk = u - row * cpr;
    } else {
      const unsigned uu = (unsigned)u;
      row = uu / cpr;
      chunk = uu - (unsigned)row * cpr;
    }
    const long long off = chunk * 16;
    const long long valid = row_bytes - off;        // bytes of the chunk inside the row, >= 1
    const uintptr_t a = reinterpret_cast<uintptr_t>(src + row * pitch + off);
    const uintptr_t g = a & ~(uintptr_t)15;
    const int s = (int)(a & 15);
    typedef const __attribute__((address_space(1))) u32x4 GlobalVec;   // global, not flat, loads
    const u32x4 lo = *reinterpret_cast<GlobalVec *>(g);
    u32x4 hi = u32x4{0u, 0u, 0u, 0u};
    if (s != 0 && (long long)(g + 16 - a) < valid) hi = *reinterpret_cast<GlobalVec *>(g + 16);
    // The chunk is bytes s .. s+15 of the 32 bytes lo, hi: first shift by
    // whole dwords (s / 4, two select stages on its bits, so that no
    // per-lane index into registers is needed), then by s % 4 bytes.
    const bool q1 = (s & 4) != 0, q2 = (s & 8) != 0;
    const uint32_t d0 = lo[0], d1 = lo[1], d2 = lo[2], d3 = lo[3];
    const uint32_t d4 = hi[0], d5 = hi[1], d6 = hi[2], d7 = hi[3];
    // e[k] = d[k + (q1 ? 1 : 0)], then f[k] = e[k + (q2 ? 2 : 0)], k = 0..4
    const uint32_t e0 = q1 ? d1 : d0, e1 = q1 ? d2 : d1, e2 = q1 ? d3 : d2, e3 = q1 ? d4 : d3;
    const uint32_t e4 = q1 ? d5 : d4, e5 = q1 ? d6 : d5, e6 = q1 ? d7 : d6;
    const uint32_t f[5] = {q2 ? e2 : e0, q2 ? e3 : e1, q2 ? e4 : e2, q2 ? e5 : e3, q2 ? e6 : e4};
    const int r = s & 3;
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = r == 0 ? f[i] : __builtin_amdgcn_alignbyte(f[i + 1], f[i], (uint32_t)r);
      if (4 * i >= valid) v = 0u;
      else if (4 * i + 4 > valid) v &= 0xffffu;     // fp16: one half of this dword is in the row
      w[i] = v;
    }
    *reinterpret_cast<u32x4 *>(dst + u * 16) = w;
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

long long ws_available(const Call &c) {
  if (c.ws_fixed != nullptr || c.ws_fixed_bytes > 0) return (long long)c.ws_fixed_bytes;
  if (c.ws_limit >= 0) return c.ws_limit < kPoolCallCap ? c.ws_limit : kPoolCallCap;
  return kPoolCallCap;
}

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
    const unsigned cpr = (unsigned)((long long)pk.lda * eb / 16);
    ja = PackJob{static_cast<const char *>(c.A), base, (long long)c.lda * eb, (long long)cols * eb,
                 cpr, (long long)rows * cpr};
    in.A = base;
    in.lda = pk.lda;
  }
  if (pk.b) {
    int rows, cols;
    stored_b(c, &rows, &cols);
    char *dst = base + pk.a_bytes;
    const unsigned cpr = (unsigned)((long long)pk.ldb * eb / 16);
    jb = PackJob{static_cast<const char *>(c.B), dst, (long long)c.ldb * eb, (long long)cols * eb,
                 cpr, (long long)rows * cpr};
    in.B = dst;
    in.ldb = pk.ldb;
  }
  // The GEMM's own workspace (split K) is the rest of the allocation.
  in.ws_fixed = base + pk.a_bytes + pk.b_bytes;
  in.ws_fixed_bytes = pk.bytes - pk.a_bytes - pk.b_bytes;
  const long long total = ja.n + jb.n;
  long long blocks = (total + kPackThreads - 1) / kPackThreads;
  if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
  if (blocks < 1) blocks = 1;
  const dim3 g((unsigned)blocks), b(kPackThreads);
  if (ja.n >= (1LL << 32) || jb.n >= (1LL << 32))
    hipLaunchKernelGGL(pack_rows<true>, g, b, 0, c.stream, ja, jb);
  else
    hipLaunchKernelGGL(pack_rows<false>, g, b, 0, c.stream, ja, jb);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch(in);
  const hipError_t f = workspace_free(c, ws);
  return e != hipSuccess ? e : f;
}

}  // namespace dgemm
