// Gram matrix of the factored norm for bf16 layers: G = A A^T, r x r, over
// K = d_in (Scaling DoRA summary page, English abstract: the Gram term
// s^2 B_i (A A^T) B_i^T of the row norm).
//
// G is small (r x r) with a long K, so its work is spread over many K splits:
// each workgroup computes one 64 x 64 tile of the upper triangle (G is
// symmetric) over one K chunk and writes it as a float32 partial sum.  Its
// four waves each own a 32 x 32 block.  Operands reach LDS by buffer loads
// straight into LDS (eight 128-byte row pieces per wave instruction, the
// 16-byte chunks of a row XOR-swizzled by the row, as in the GEMM) through a
// ring of four 64-deep stages: a workgroup has only a few stages of work, so
// keeping several in flight hides the copies' latency, which a two-stage
// pipeline would expose once per stage.
//
// The finisher adds the partial sums of each element in split order (fixed,
// so the result is bitwise reproducible) and writes each upper-triangle value
// to both of its places (so the result is exactly symmetric, and the
// projection may use G's rows as its columns), scaled by s/2, as a bf16 hi + lo
// pair (hi = round(v),
// lo = round(v - hi)) that carries ~16 significant bits through the bf16
// MFMA.  It also clears a region of counters that later kernels of the same
// call use.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dora {
namespace {

constexpr int kGT = 64;          // tile edge
constexpr int kGK = 64;          // K depth of one stage
constexpr int kGRowB = kGK * 2;  // bytes of one row piece
constexpr int kGRing = 4;        // stages in flight
constexpr int kGStageB = 2 * kGT * kGRowB;   // A-side then B-side rows: 16 KiB

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane((int)b),
                                           0x00020000);
}

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// s_waitcnt vmcnt(N) with the other counters left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Upper-triangle tile t of an n x n tile grid -> (ti, tj), ti <= tj, row by row.
__device__ __forceinline__ void tri_tile(int t, int n, int& ti, int& tj) {
  int row = 0, first = 0;
  while (t >= first + (n - row)) {
    first += n - row;
    ++row;
  }
  ti = row;
  tj = row + (t - first);
}

// part[(tile * splits + split) * 64 * 64 + a * 64 + b] = sum over the split's K
// chunk of A[ti*64 + a, k] * A[tj*64 + b, k].
__global__ __launch_bounds__(256) void dora_gram_partial(const uint16_t* A, int r, int d_in,
                                                         int kchunk, float* part) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[kGRing * kGStageB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = (r + kGT - 1) / kGT;
  int ti, tj;
  tri_tile(blockIdx.x, nt, ti, tj);
  const int k_lo = blockIdx.y * kchunk;
  const int k_hi = min(d_in, k_lo + kchunk);
  const int nst = (k_hi - k_lo + kGK - 1) / kGK;
  const bool tail = (k_hi - k_lo) % kGK != 0;   // only the very last chunk of A's K can be partial
  const Rsrc rs = rsrc(A, (int64_t)r * d_in * 2);
  // Copy instruction q of this wave fills LDS rows (wave + 4q) * 8 .. + 8 of a
  // stage: rows 0-63 are the A-side tile rows, 64-127 the B-side ones.  Rows
  // past r read zeros (offset beyond the records); the K position of a stage
  // travels in the scalar offset and stays inside the row.
  uint32_t off[4];
  int lc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int R = (wave + 4 * q) * 8 + (lane >> 3);
    const int gr = (R < kGT ? ti : tj) * kGT + (R & (kGT - 1));
    lc[q] = (lane & 7) ^ swz(R);
    off[q] = gr < r ? (uint32_t)gr * (uint32_t)(d_in * 2) + (uint32_t)lc[q] * 16u : kOob;
  }
  auto issue = [&](int st) {
    uint8_t* dst = sm + (st % kGRing) * kGStageB;
    const int k0 = k_lo + st * kGK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t o = off[q];
      if (tail && st == nst - 1 && k0 + lc[q] * 8 >= k_hi) o = kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (wave + 4 * q) * 8 * kGRowB), 16,
          (int)o, k0 * 2, 0, 0);
    }
  };
  const int pre = min(kGRing, nst);
  for (int st = 0; st < pre; ++st) issue(st);

  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const int ra = (wave & 1) * 32 + (lane & 31);            // A-side LDS row
  const int rb = kGT + (wave >> 1) * 32 + (lane & 31);     // B-side LDS row
  for (int st = 0; st < nst; ++st) {
    // stage st has landed once at most the copies of the stages issued after it
    // are still in flight (4 instructions per stage and wave)
    const int later = min(kGRing - 1, nst - 1 - st);
    if (later >= 3) wait_vm<12>();
    else if (later == 2) wait_vm<8>();
    else if (later == 1) wait_vm<4>();
    else wait_vm<0>();
    barrier_nofence();
    const uint8_t* src = sm + (st % kGRing) * kGStageB;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      fa[kk] = *reinterpret_cast<const bf16x8*>(src + ra * kGRowB + ((ch ^ swz(ra)) << 4));
      fb[kk] = *reinterpret_cast<const bf16x8*>(src + rb * kGRowB + ((ch ^ swz(rb)) << 4));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk], fa[kk], acc, 0, 0, 0);
    barrier_nofence();   // every wave has read the slot before it is refilled
    if (st + kGRing < nst) issue(st + kGRing);
  }
  // acc[v]: row a = lane % 32 of the A-side block, column (v/4)*8 + (lane/32)*4 + v%4
  // of the B-side block
  float* dst = part + ((int64_t)blockIdx.x * gridDim.y + blockIdx.y) * kGT * kGT;
  const int a = (wave & 1) * 32 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int b = (wave >> 1) * 32 + g * 8 + (lane >> 5) * 4;
    *reinterpret_cast<f32x4*>(dst + a * kGT + b) =
        f32x4{acc[g * 4], acc[g * 4 + 1], acc[g * 4 + 2], acc[g * 4 + 3]};
  }
}

// Workgroup (tile, g) finishes rows 4g .. 4g + 3 of an upper-triangle tile: each
// thread adds one element's split sums in split order (coalesced, every load in
// flight before the first add; at most kGMaxSplits splits) and writes the scaled
// hi + lo pair at (i, j) and at the mirror (j, i).  On a diagonal tile only the
// elements on or above the diagonal are taken, each written to both places, so
// G comes out exactly symmetric.
constexpr int kGFinRows = 4;
constexpr int kGMaxSplits = 32;
__global__ __launch_bounds__(256) void dora_gram_finish(const float* part, int splits, int r,
                                                        float scale, uint16_t* g_hi,
                                                        uint16_t* g_lo, uint32_t* zero,
                                                        int64_t nzero) {
  const int tid = threadIdx.x;
  const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
  const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  for (int64_t i = wg * 256 + tid; i < nzero; i += nwg * 256) zero[i] = 0u;
  const int nt = (r + kGT - 1) / kGT;
  int ti, tj;
  tri_tile(blockIdx.x, nt, ti, tj);
  const int a = blockIdx.y * kGFinRows + tid / kGT, b = tid % kGT;
  if (ti == tj && a > b) return;
  const int i = ti * kGT + a, j = tj * kGT + b;
  if (i >= r || j >= r) return;
  const float* p = part + (int64_t)blockIdx.x * splits * kGT * kGT + a * kGT + b;
  constexpr int64_t kS = kGT * kGT;
  float part_v[kGMaxSplits];
#pragma unroll
  for (int u = 0; u < kGMaxSplits; ++u) part_v[u] = u < splits ? p[u * kS] : 0.f;
  float s = part_v[0];
#pragma unroll
  for (int u = 1; u < kGMaxSplits; ++u)
    if (u < splits) s += part_v[u];
  const float v = scale * s;
  const uint16_t hi = f32_to_bf16(v);
  const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
  g_hi[(int64_t)i * r + j] = hi;
  g_lo[(int64_t)i * r + j] = lo;
  if (i != j) {
    g_hi[(int64_t)j * r + i] = hi;
    g_lo[(int64_t)j * r + i] = lo;
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

GramPlan gram_bf16_plan(int64_t r, int64_t d_in) {
  GramPlan g{};
  const int64_t nt = cdiv(r, kGT);
  g.tiles = nt * (nt + 1) / 2;
  // At most about 256 workgroups, so that no CU takes two; K chunks a whole
  // number of stages.  Measured at r = 384, d_in = 8192 (21 tiles): 12 chunks
  // (252 workgroups) 10.5 us, 16 chunks (336) 12.2 us, 22 chunks (462) 11.7 us.
  const int64_t span = kGK;
  // (at most kGMaxSplits: the finisher holds every split of an element at once)
  int64_t splits = std::max<int64_t>(1, std::min<int64_t>(kGMaxSplits, 256 / g.tiles));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, cdiv(d_in, span)));
  g.kchunk = cdiv(cdiv(d_in, splits), span) * span;
  g.splits = cdiv(d_in, g.kchunk);
  g.part_bytes = (size_t)g.tiles * g.splits * kGT * kGT * 4;
  return g;
}

hipError_t gram_bf16(const void* A, int64_t r, int64_t d_in, const GramPlan& g, float* part,
                     hipStream_t st) {
  if (r <= 0) return hipSuccess;
  LaunchTimer t("gram_AAt", st);
  hipLaunchKernelGGL(dora_gram_partial, dim3((unsigned)g.tiles, (unsigned)g.splits), dim3(256), 0,
                     st, reinterpret_cast<const uint16_t*>(A), (int)r, (int)d_in, (int)g.kchunk,
                     part);
  return hipGetLastError();
}

hipError_t gram_bf16_finish(const float* part, const GramPlan& g, int64_t r, float scale,
                            void* g_hi, void* g_lo, uint32_t* zero, int64_t nzero,
                            hipStream_t st) {
  if (r <= 0) return hipSuccess;
  LaunchTimer t("gram_finalize", st);
  hipLaunchKernelGGL(dora_gram_finish, dim3((unsigned)g.tiles, kGT / kGFinRows), dim3(256), 0, st,
                     part,
                     (int)g.splits, (int)r, scale, reinterpret_cast<uint16_t*>(g_hi),
                     reinterpret_cast<uint16_t*>(g_lo), zero, nzero);
  return hipGetLastError();
}

}  // namespace dora
