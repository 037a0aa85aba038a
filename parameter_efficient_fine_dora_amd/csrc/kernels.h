// Internal interface between the C ABI (api.hip) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace dora {

enum DType : int { kF32 = 0, kBF16 = 1 };

// One K segment of C += op(A) op(B)^T.  Element (m, k) of op(A) is
// a[m*lda + k] when the A operand is K-contiguous, a[k*lda + m] otherwise;
// element (n, k) of op(B) likewise with b / ldb.
struct GemmSeg {
  const void* a;
  const void* b;
  int64_t lda, ldb;
  int64_t K;
};

enum Epilogue : int {
  kEpiStore = 0,     // C = alpha * acc
  kEpiCompose = 1,   // C = z + (g - 1) z with z = alpha * acc, g_n = m_n / max(norm_n, eps)
  kEpiMerge = 2,     // C = g_m (add + alpha * acc) with g_m = m_m / max(norm_m, eps) per ROW
  kEpiNorm = 3,      // C is not stored; rowsq[z][m] = sum over segment 0 of opA(m, k)^2
                     // and rowdot[z][tile_n][m] = alpha * sum over the tile's
                     // n of C(m, n) * add(m, n) (bf16, both operands K-contiguous;
                     // z = split index)
};

struct GemmProblem {
  int64_t M = 0, N = 0;
  int nseg = 0;
  GemmSeg seg[3] = {};
  bool a_kcontig = true, b_kcontig = true;   // same for every segment
  void* c = nullptr;
  int64_t ldc = 0;
  float alpha = 1.f;
  bool out_f32 = false;        // C is float32 (else the layer dtype)
  int split = 1;               // split-K factor: C_z written at c + z*split_stride
  int64_t split_stride = 0;    // elements
  int epi = kEpiStore;
  const void* mag = nullptr;   // kEpiCompose: m [N]; kEpiMerge: m [M] (layer dtype)
  const float* norm = nullptr; // kEpiCompose: n [N]; kEpiMerge: n [M] (float32)
  const void* add = nullptr;   // kEpiMerge: addend [M, N] (layer dtype), row stride ld_add
  int64_t ld_add = 0;
  float* rowsq = nullptr;      // kEpiNorm: [split][M] float32 partial row sums of squares
  float* rowdot = nullptr;     // kEpiNorm: [gemm_col_slots * split][M] float32 partial row dots
  float* norm_out = nullptr;   // kEpiNorm: if set, the row norms sqrt(max(0, sum rowsq + sum
                               // rowdot)), formed by the last workgroup of each tile row
  uint32_t* done = nullptr;    // kEpiNorm with norm_out: gemm_tile_rows counters, zero at launch
  // Library-chosen split-K (layer-dtype store epilogue only): float32 partial
  // sums go to `scratch`, then a fixed-order reduction writes C.
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  int cfg = -1;                // tile configuration override (-1 = planner's choice)
  int force_split = 0;         // split-K override for the scratch path (0 = planner's choice)
};

struct GemmPlan {
  int cfg;     // tile configuration index (-1: the float32 kernel)
  int split;   // split-K factor
};

// Tile configuration and split-K factor for a layer-dtype GEMM of this size
// and operand layout.
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int dtype, bool akc = true, bool bkc = true);

// Tile configuration and split-K factor of the norm's projection P = [W0 | B | B] [A | G]^T
// (M = d_out, N = r, K = d_in + 2r; ld_max = the largest row stride of its operands).
GemmPlan plan_norm_projection(int64_t M, int64_t N, int64_t K, int64_t ld_max);

// Tile-rows of a GEMM with M rows on tile configuration cfg.
int64_t gemm_tile_rows(int cfg, int64_t M);

// Row-dot partials per split of a kEpiNorm GEMM with N columns on tile configuration cfg.
int64_t gemm_col_slots(int cfg, int64_t N);

// Scratch bytes the split-K path of gemm() needs for this problem (0 if unsplit).
size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K, int dtype, bool akc = true,
                          bool bkc = true);

// Enqueue C = sum over segments; picks the tile configuration from the shape.
hipError_t gemm(const GemmProblem& p, int dtype, hipStream_t st, const char* label);


// Gram matrix G = A A^T of a bf16 A [r, d_in] (csrc/gram.hip): float32 partial
// sums of the upper-triangle 64 x 64 tiles over K splits, then a finisher that
// writes scale * G as a bf16 hi + lo pair (exactly symmetric) and zeroes
// `nzero` counters for later kernels of the call.
struct GramPlan {
  int64_t tiles;       // upper-triangle tiles
  int64_t splits;      // K chunks
  int64_t kchunk;      // K extent of one chunk
  size_t part_bytes;   // float32 partial sums
};
GramPlan gram_bf16_plan(int64_t r, int64_t d_in);
hipError_t gram_bf16(const void* A, int64_t r, int64_t d_in, const GramPlan& g, float* part,
                     hipStream_t st);
hipError_t gram_bf16_finish(const float* part, const GramPlan& g, int64_t r, float scale,
                            void* g_hi, void* g_lo, uint32_t* zero, int64_t nzero,
                            hipStream_t st);

// scale * (sum of r x r partial sums); bf16: written as a hi + lo bf16 pair.
hipError_t gram_finalize(const float* part, int splits, int64_t r, float scale, int dtype,
                         void* g_hi, void* g_lo, hipStream_t st, const char* label);

// Undetached norm gradient: k'_i = -s m_i dm_i / n_i^2 (float32) and Bk' = diag(k') B.
hipError_t exact_prep(const void* m, const float* norm, const float* dm, const void* B, float s,
                      float* kappa, void* Bk, int64_t d_out, int64_t r, int dtype,
                      hipStream_t st);

// dB = sum of d1 partials + k'_i * (sum of q partials), [d_out, r].
// DVoRA: B_eff = diag(b) B_sh diag(d); db, dd from grad_B_eff (dd through
// vera_dd_blocks(d_out) float32 row-block partials of r columns in `part`).
hipError_t vera_scale(const void* Bsh, const void* b, const void* d, void* Be, int64_t d_out,
                      int64_t r, int dtype, hipStream_t st);
int64_t vera_dd_blocks(int64_t d_out);
hipError_t vera_grads(const void* gBe, const void* Bsh, const void* b, const void* d, void* db,
                      void* dd, float* part, int64_t d_out, int64_t r, int dtype, hipStream_t st);

hipError_t db_combine(const float* d1, int d1_splits, const float* q, int q_splits,
                      const float* kappa, void* dB, int64_t d_out, int64_t r, int dtype,
                      hipStream_t st);

// n_i = sqrt(max(0, ||W0_i||^2 + B_i . P_i)), P = sum of p_splits partials
// [p_splits][d_out][r] (float32), ||W0_i||^2 streamed from W0.
hipError_t row_norm(const void* W0, const void* B, const float* P, int p_splits, float* norm,
                    int64_t d_out, int64_t d_in, int64_t r, int dtype, hipStream_t st);

// y = base + ((g-1) base + g * slora) in place on y (base), slora = s * lora.
hipError_t compose_fwd(void* y, const void* slora, const void* m, const float* norm, int64_t T,
                       int64_t d_out, int dtype, hipStream_t st);

// gz = g * gy; dm_part[b, i] = sum over token block b of gy * y.
hipError_t compose_bwd(const void* gy, const void* y, const void* m, const float* norm, void* gz,
                       float* dm_part, int64_t T, int64_t d_out, int64_t tokens_per_block,
                       int dtype, hipStream_t st);

// Bg^T = (s diag(g) B)^T, [r, d_out], g_i = m_i / max(n_i, eps), in the layer dtype.
hipError_t scale_b_rows_t(const void* B, const void* m, const float* norm, float s, void* Bgt,
                          int64_t d_out, int64_t r, int dtype, hipStream_t st);

// What dm_finalize needs to recompute a column whose m_i is zero (where
// y / m = z / n does not hold): dm_i = sum_t gy[t,i] (x_t . (W0_i + s B_i A)) / n_i.
struct DmRecompute {
  const float* norm;
  const void *gy, *x, *W0, *A, *B;
  float s;
  int64_t T, d_in, r;
};

// dm_i = sum_b dm_part[b, i] / m_i (fixed order); columns with m_i == 0 from `z`.
hipError_t dm_finalize(const float* dm_part, int64_t blocks, const void* m, float* dm,
                       int64_t d_out, const DmRecompute& z, int dtype, hipStream_t st);

// The whole forward of a small float32 layer in two kernels (csrc/small.hip):
// norm, y and xs for tokens <= kSmallMaxTokens, r <= kSmallMaxRank,
// d_in <= kSmallMaxDin, d_out <= kSmallMaxDout.  The first kernel splits K into
// `ksplits` ranges of `chunks` 64-deep chunks over `row_blocks` blocks of 16
// output rows and writes float32 partial sums to `part`; the second sums them
// in split order and applies the norm and the compose.
constexpr int kSmallMaxTokens = 64;
constexpr int kSmallMaxRank = 32;
constexpr int64_t kSmallMaxDin = 1024;
constexpr int64_t kSmallMaxDout = 4096;
struct SmallPlan {
  int64_t row_blocks, ksplits, chunks;
  size_t part_bytes;
};
inline bool small_forward_fits(int64_t T, int64_t d_out, int64_t d_in, int64_t r) {
  return T >= 1 && T <= kSmallMaxTokens && r >= 0 && r <= kSmallMaxRank && d_in >= 1 &&
         d_in <= kSmallMaxDin && d_out >= 1 && d_out <= kSmallMaxDout;
}
inline SmallPlan small_forward_plan(int64_t d_out, int64_t d_in) {
  SmallPlan p;
  p.row_blocks = (d_out + 15) / 16;
  const int64_t nchunk = (d_in + 63) / 64;
  // up to 256 workgroups where the row blocks alone leave the chip idle
  const int64_t want = std::min<int64_t>(nchunk, std::max<int64_t>(1, 256 / p.row_blocks));
  p.chunks = (nchunk + want - 1) / want;
  p.ksplits = (nchunk + p.chunks - 1) / p.chunks;
  // per (split, row block): z [64][16] and U | ||W0_i||^2 [16][33];
  // per split: x A^T [64][32] and A A^T [32][32]
  p.part_bytes = (size_t)p.ksplits * ((size_t)p.row_blocks * (64 * 16 + 16 * 33) + 64 * 32 + 32 * 32) * 4;
  return p;
}
hipError_t small_forward(const float* x, const float* W0, const float* A, const float* B,
                         const float* m, float s, float* y, float* norm, float* xs, float* part,
                         int64_t T, int64_t d_out, int64_t d_in, int64_t r, hipStream_t st);

// Launch bookkeeping for the optional per-kernel timing.
struct LaunchTimer {
  LaunchTimer(const char* label, hipStream_t st);
  ~LaunchTimer();
  const char* label_;
  hipStream_t st_;
  void* ev_[2];
};

}  // namespace dora
