// Bandwidth-bound kernels of the DoRA hot path on gfx950: the Gram finisher,
// the factored row norm, and the standalone compose forward / backward.
// Every tensor is streamed with 16-byte vector loads along its contiguous
// dimension (8 bf16 or 4 float32 per load), accumulation is float32.
#include "kernels.h"
#include "common.h"

namespace dora {
namespace {

template <bool BF>
struct Vec;   // one 16-byte vector of the layer dtype
template <>
struct Vec<true> {
  static constexpr int kN = 8;
  __device__ static void load(const void* p, int64_t i, float* out) {   // i in vectors
    const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      out[2 * d] = bf_lo(v[d]);
      out[2 * d + 1] = bf_hi(v[d]);
    }
  }
  __device__ static void store(void* p, int64_t i, const float* in) {
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = pack_bf16x2(in[2 * d], in[2 * d + 1]);
    reinterpret_cast<u32x4*>(p)[i] = v;
  }
  __device__ static float scalar(const void* p, int64_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
};
template <>
struct Vec<false> {
  static constexpr int kN = 4;
  __device__ static void load(const void* p, int64_t i, float* out) {
    const f32x4 v = reinterpret_cast<const f32x4*>(p)[i];
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = v[d];
  }
  __device__ static void store(void* p, int64_t i, const float* in) {
    reinterpret_cast<f32x4*>(p)[i] = f32x4{in[0], in[1], in[2], in[3]};
  }
  __device__ static float scalar(const void* p, int64_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- Gram finisher ------------------------------------------------------------
// part[z], z < splits: split-K partial sums of G = A A^T, added in a fixed
// order.  Writes (s/2) G; bf16 layers get it as a hi + lo bf16 pair
// (hi = round(v), lo = round(v - hi)), which keeps ~16 significant bits through
// the bf16 MFMA.  G is symmetric (up to the rounding of its partial sums), so
// the projection may use its rows for its columns.
__global__ __launch_bounds__(256) void dora_gram_finalize(const float* part, int splits,
                                                          int64_t rr, float half_s, int bf,
                                                          void* g_hi, void* g_lo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rr) return;
  const float v = half_s * sum_partials(part + idx, splits, rr);
  if (bf) {
    const uint16_t hi = f32_to_bf16(v);
    const float rest = v - bf16_to_f32(hi);
    reinterpret_cast<uint16_t*>(g_hi)[idx] = hi;
    reinterpret_cast<uint16_t*>(g_lo)[idx] = f32_to_bf16(rest);
  } else {
    reinterpret_cast<float*>(g_hi)[idx] = v;
  }
}

// ---- factored row norm --------------------------------------------------------
// One wave per output row i:
//   n_i^2 = sum_k W0_ik^2 + sum_j B_ij P_ij,   P = 2s W0 A^T + s^2 B G,
// i.e. base + cross + Gram.  W0's row is streamed once with 16-byte loads,
// four in flight per lane; B_i and P_i are read once each (no reuse, so they
// go straight to registers) and the lane partials meet in a wave reduction.
template <bool BF>
__global__ __launch_bounds__(256) void dora_row_norm(const void* W0, const void* B, const float* P,
                                                     int p_splits, int64_t p_stride, float* norm,
                                                     int64_t d_out, int64_t d_in, int64_t r) {
  using V = Vec<BF>;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= d_out) return;   // whole wave leaves; the kernel has no barrier
  const int64_t nv = d_in / V::kN;
  const int64_t wbase = row * nv;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  int64_t c = lane;
  for (; c + 192 < nv; c += 256) {
    float a[V::kN], b[V::kN], e[V::kN], f[V::kN];
    V::load(W0, wbase + c, a);
    V::load(W0, wbase + c + 64, b);
    V::load(W0, wbase + c + 128, e);
    V::load(W0, wbase + c + 192, f);
#pragma unroll
    for (int q = 0; q < V::kN; ++q) {
      acc0 = fmaf(a[q], a[q], acc0);
      acc1 = fmaf(b[q], b[q], acc1);
      acc2 = fmaf(e[q], e[q], acc2);
      acc3 = fmaf(f[q], f[q], acc3);
    }
  }
  for (; c < nv; c += 64) {
    float a[V::kN];
    V::load(W0, wbase + c, a);
#pragma unroll
    for (int q = 0; q < V::kN; ++q) acc0 = fmaf(a[q], a[q], acc0);
  }
  // cross + Gram: B_i . P_i, P given as p_splits split-K partial sums
  const int64_t rv = r / V::kN;
  const float* prow = P + row * r;
  for (int64_t cc = lane; cc < rv; cc += 64) {
    float bv[V::kN];
    V::load(B, row * rv + cc, bv);
#pragma unroll
    for (int q = 0; q < V::kN; q += 4) {
      f32x4 pv = *reinterpret_cast<const f32x4*>(prow + cc * V::kN + q);
      for (int z = 1; z < p_splits; ++z)
        pv += *reinterpret_cast<const f32x4*>(prow + z * p_stride + cc * V::kN + q);
      acc1 = fmaf(bv[q], pv[0], acc1);
      acc1 = fmaf(bv[q + 1], pv[1], acc1);
      acc1 = fmaf(bv[q + 2], pv[2], acc1);
      acc1 = fmaf(bv[q + 3], pv[3], acc1);
    }
  }
  const float tot = wave_sum((acc0 + acc1) + (acc2 + acc3));
  if (lane == 0) norm[row] = sqrtf(fmaxf(tot, 0.f));
}

// ---- compose forward ------------------------------------------------------------
// y = base + ((g - 1) base + g * slora), base read from y and overwritten,
// slora = s (x A^T) B^T, g - 1 = (m - n) / n with n clamped at kNormEps,
// everything in float32 and rounded once.  Thread = one 16-byte column vector,
// looping over a block of tokens; g and g - 1 are formed once per thread.
template <bool BF>
__global__ __launch_bounds__(256) void dora_compose_fwd(void* y, const void* slora, const void* m,
                                                        const float* norm, int64_t T,
                                                        int64_t d_out, int64_t tok_per_block) {
  using V = Vec<BF>;
  const int64_t nvec = d_out / V::kN;
  const int64_t cv = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (cv >= nvec) return;
  float g[V::kN], gm1[V::kN];
#pragma unroll
  for (int q = 0; q < V::kN; ++q) {
    const int64_t col = cv * V::kN + q;
    const float n = fmaxf(norm[col], kNormEps);
    const float mv = V::scalar(m, col);
    gm1[q] = (mv - n) / n;
    g[q] = mv / n;
  }
  const int64_t t0 = (int64_t)blockIdx.y * tok_per_block;
  const int64_t t1 = min(T, t0 + tok_per_block);
  constexpr int U = 4;   // tokens in flight per thread
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
    float base[U][V::kN], lo[U][V::kN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      V::load(y, (t + u) * nvec + cv, base[u]);
      V::load(slora, (t + u) * nvec + cv, lo[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float out[V::kN];
#pragma unroll
      for (int q = 0; q < V::kN; ++q)
        out[q] = base[u][q] + fmaf(gm1[q], base[u][q], g[q] * lo[u][q]);
      V::store(y, (t + u) * nvec + cv, out);
    }
  }
  for (; t < t1; ++t) {
    float base[V::kN], lo[V::kN], out[V::kN];
    V::load(y, t * nvec + cv, base);
    V::load(slora, t * nvec + cv, lo);
#pragma unroll
    for (int q = 0; q < V::kN; ++q) out[q] = base[q] + fmaf(gm1[q], base[q], g[q] * lo[q]);
    V::store(y, t * nvec + cv, out);
  }
}

// ---- compose backward -------------------------------------------------------------
// With the norm detached (held constant), y = g z gives dL/dz = g * gy and
// dL/dm_i = sum_t gy[t,i] z[t,i] / n_i = sum_t gy[t,i] y[t,i] / m_i.
// This kernel writes gz = g * gy and, per token block b, the column partial
// sums dm_part[b, i] = sum_{t in b} gy[t,i] y[t,i]; dora_dm_finalize adds the
// blocks in a fixed order, so the result does not depend on scheduling.
template <bool BF>
__global__ __launch_bounds__(256) void dora_compose_bwd(const void* gy, const void* y,
                                                        const void* m, const float* norm, void* gz,
                                                        float* dm_part, int64_t T, int64_t d_out,
                                                        int64_t tok_per_block) {
  using V = Vec<BF>;
  const int64_t nvec = d_out / V::kN;
  const int64_t cv = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (cv >= nvec) return;
  float g[V::kN], acc[V::kN];
#pragma unroll
  for (int q = 0; q < V::kN; ++q) {
    const int64_t col = cv * V::kN + q;
    g[q] = V::scalar(m, col) / fmaxf(norm[col], kNormEps);
    acc[q] = 0.f;
  }
  const int64_t t0 = (int64_t)blockIdx.y * tok_per_block;
  const int64_t t1 = min(T, t0 + tok_per_block);
  constexpr int U = 4;   // tokens in flight per thread
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
    float a[U][V::kN], b[U][V::kN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      V::load(gy, (t + u) * nvec + cv, a[u]);
      V::load(y, (t + u) * nvec + cv, b[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float o[V::kN];
#pragma unroll
      for (int q = 0; q < V::kN; ++q) {
        o[q] = g[q] * a[u][q];
        acc[q] = fmaf(a[u][q], b[u][q], acc[q]);
      }
      V::store(gz, (t + u) * nvec + cv, o);
    }
  }
  for (; t < t1; ++t) {
    float a[V::kN], b[V::kN], o[V::kN];
    V::load(gy, t * nvec + cv, a);
    V::load(y, t * nvec + cv, b);
#pragma unroll
    for (int q = 0; q < V::kN; ++q) {
      o[q] = g[q] * a[q];
      acc[q] = fmaf(a[q], b[q], acc[q]);
    }
    V::store(gz, t * nvec + cv, o);
  }
  float* dst = dm_part + (int64_t)blockIdx.y * d_out + cv * V::kN;
#pragma unroll
  for (int q = 0; q < V::kN; q += 4)
    *reinterpret_cast<f32x4*>(dst + q) = f32x4{acc[q], acc[q + 1], acc[q + 2], acc[q + 3]};
}

// 64 columns per workgroup, the partial blocks split over 4 thread rows and
// combined through LDS in a fixed order.
//
// dm_i = (sum_t gy[t,i] y[t,i]) / m_i rests on y / m = z / n, which says
// nothing when m_i = 0 (column i of y is then 0 and carries no z).  Such a
// column is recomputed from the definition, dm_i = sum_t gy[t,i] z[t,i] / n_i
// with z[t,i] = x_t . V'_i and V'_i = W0_i + s B_i A: the workgroup's threads
// share d_in, each forms its V'_ik and sum_t gy[t,i] x[t,k], and the products
// meet in a fixed-order LDS reduction.  It costs T * (d_in + r) reads per zero
// column and nothing when no m_i of the workgroup is zero.
template <bool BF>
__global__ __launch_bounds__(256) void dora_dm_finalize(
    const float* dm_part, int64_t blocks, const void* m, float* dm, int64_t d_out,
    const float* norm, const void* gy, const void* x, const void* W0, const void* A,
    const void* B, float s_lora, int64_t T, int64_t d_in, int64_t r) {
  using V = Vec<BF>;
  __shared__ float red[4][64];
  __shared__ float tree[256];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + c;
  float s = 0.f;
  if (i < d_out && q < blocks) s = sum_partials(dm_part + q * d_out + i, (blocks - q + 3) / 4, 4 * d_out);
  red[q][c] = s;
  const bool zero_m = q == 0 && i < d_out && V::scalar(m, i) == 0.f;
  if (!__syncthreads_or(zero_m)) {
    if (q == 0 && i < d_out)
      dm[i] = ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c])) / V::scalar(m, i);
    return;
  }
  if (q == 0 && i < d_out && !zero_m)
    dm[i] = ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c])) / V::scalar(m, i);
  for (int cc = 0; cc < 64; ++cc) {
    const int64_t col = (int64_t)blockIdx.x * 64 + cc;
    if (col >= d_out) break;
    if (V::scalar(m, col) != 0.f) continue;   // the same test in every thread
    float acc = 0.f;
    for (int64_t k = threadIdx.x; k < d_in; k += 256) {
      float ba = 0.f;
      for (int64_t j = 0; j < r; ++j) ba = fmaf(V::scalar(B, col * r + j), V::scalar(A, j * d_in + k), ba);
      const float v = fmaf(s_lora, ba, V::scalar(W0, col * d_in + k));
      float gx = 0.f;
      for (int64_t t = 0; t < T; ++t)
        gx = fmaf(V::scalar(gy, t * d_out + col), V::scalar(x, t * d_in + k), gx);
      acc = fmaf(v, gx, acc);
    }
    tree[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h) tree[threadIdx.x] += tree[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) dm[col] = tree[0] / fmaxf(norm[col], kNormEps);
    __syncthreads();
  }
}

// ---- undetached norm gradient (Appendix A.1 of the DoRA reading notes) -----------
// Projecting dW'_i off V'_i adds -kappa_i V'_i to dV'_i with
// kappa_i = m_i dm_i / n_i^2 (since dW'_i . V'_i = dm_i n_i).  Through
// V' = W0 + s B A that gives dB_i += k'_i (W0 A^T + s B G)_i and
// dA += Bk'^T W0 + s (Bk'^T B) A, with k' = -s kappa and Bk' = diag(k') B.
// This kernel forms k' (float32) and Bk' (layer dtype).
template <bool BF>
__global__ __launch_bounds__(256) void dora_exact_prep(const void* m, const float* norm,
                                                       const float* dm, const void* B, float s,
                                                       float* kappa, void* Bk, int64_t d_out,
                                                       int64_t r) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = r > 0 ? idx / r : idx;
  if (i >= d_out) return;
  const float n = fmaxf(norm[i], kNormEps);
  const float kp = -s * Vec<BF>::scalar(m, i) * dm[i] / (n * n);
  if (r == 0 || idx % r == 0) kappa[i] = kp;
  if (r > 0) {
    const float b = Vec<BF>::scalar(B, idx);
    if (BF)
      reinterpret_cast<uint16_t*>(Bk)[idx] = f32_to_bf16(kp * b);
    else
      reinterpret_cast<float*>(Bk)[idx] = kp * b;
  }
}

// Bg^T = (s diag(g) B)^T, [r, d_out], with g_i = m_i / max(n_i, eps) (float32
// product, rounded once): with it the rank-space gradient ts = s (g * gy) B is
// gy Bg, which needs only the incoming gradient (so it need not wait for the
// compose backward), and with Bg stored transposed both operands of that
// product are K-contiguous.  A workgroup moves one 64 x 64 block through LDS:
// rows of B read along r, rows of Bg^T written along d_out, both coalesced.
constexpr int kTb = 64;
template <bool BF>
__global__ __launch_bounds__(256) void dora_scale_b_rows_t(const void* B, const void* m,
                                                           const float* norm, float s, void* Bgt,
                                                           int64_t d_out, int64_t r) {
  using V = Vec<BF>;
  constexpr int kC = kTb / V::kN;   // 16-byte chunks along one 64-wide row of the block
  __shared__ float tile[kTb][kTb + 1];
  __shared__ float sg[kTb];
  const int64_t i0 = (int64_t)blockIdx.x * kTb, q0 = (int64_t)blockIdx.y * kTb;
  if (threadIdx.x < kTb) {
    const int64_t i = i0 + threadIdx.x;
    sg[threadIdx.x] = i < d_out ? s * (V::scalar(m, i) / fmaxf(norm[i], kNormEps)) : 0.f;
  }
  __syncthreads();
  // d_out and r are multiples of the vector width, so a chunk is wholly inside or outside
  for (int e = threadIdx.x; e < kTb * kC; e += 256) {
    const int il = e / kC, ql = (e % kC) * V::kN;
    const int64_t i = i0 + il, q = q0 + ql;
    if (i < d_out && q < r) {
      float v[V::kN];
      V::load(B, (i * r + q) / V::kN, v);
#pragma unroll
      for (int u = 0; u < V::kN; ++u) tile[il][ql + u] = sg[il] * v[u];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kTb * kC; e += 256) {
    const int ql = e / kC, il = (e % kC) * V::kN;
    const int64_t i = i0 + il, q = q0 + ql;
    if (i < d_out && q < r) {
      float v[V::kN];
#pragma unroll
      for (int u = 0; u < V::kN; ++u) v[u] = tile[il + u][ql];
      V::store(Bgt, (q * d_out + i) / V::kN, v);
    }
  }
}

// dB = sum_z D1_z + k'_i * sum_z Q_z, each in a fixed order, rounded once.
template <bool BF>
__global__ __launch_bounds__(256) void dora_db_combine(const float* d1, int d1_splits,
                                                       const float* q, int q_splits,
                                                       const float* kappa, void* dB, int64_t n,
                                                       int64_t r) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  float a = 0.f, b = 0.f;
  for (int z = 0; z < d1_splits; ++z) a += d1[z * n + idx];
  for (int z = 0; z < q_splits; ++z) b += q[z * n + idx];
  const float v = fmaf(kappa[idx / r], b, a);
  if (BF)
    reinterpret_cast<uint16_t*>(dB)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<float*>(dB)[idx] = v;
}

// ---- DVoRA (DoRA reading notes, Sec. 3.5) --------------------------------------
// The VeRA direction update diag(b) B_sh diag(d) A_sh enters the DoRA path as
// the effective B = diag(b) B_sh diag(d); its gradient comes back as grad_B_eff
// and splits into the two vectors:
//   db_i = sum_j grad_B_eff_ij B_sh_ij d_j,   dd_j = sum_i grad_B_eff_ij b_i B_sh_ij.

// B_eff = b_i * B_sh_ij * d_j, float32 product rounded once.
template <bool BF>
__global__ __launch_bounds__(256) void dora_vera_scale(const void* Bsh, const void* b,
                                                       const void* d, void* Be, int64_t n,
                                                       int64_t r) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const float v = Vec<BF>::scalar(b, idx / r) * Vec<BF>::scalar(Bsh, idx) *
                  Vec<BF>::scalar(d, idx % r);
  if (BF)
    reinterpret_cast<uint16_t*>(Be)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<float*>(Be)[idx] = v;
}

// db: one wave per row, lanes striding over the rank.
template <bool BF>
__global__ __launch_bounds__(256) void dora_vera_db(const void* gBe, const void* Bsh,
                                                    const void* d, void* db, int64_t d_out,
                                                    int64_t r) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= d_out) return;
  float acc = 0.f;
  for (int64_t j = lane; j < r; j += 64)
    acc += Vec<BF>::scalar(gBe, i * r + j) * Vec<BF>::scalar(Bsh, i * r + j) *
           Vec<BF>::scalar(d, j);
  acc = wave_sum(acc);
  if (lane == 0) {
    if (BF)
      reinterpret_cast<uint16_t*>(db)[i] = f32_to_bf16(acc);
    else
      reinterpret_cast<float*>(db)[i] = acc;
  }
}

// dd, stage 1: each block sums kVeraRows consecutive rows of 256 columns, in order.
constexpr int kVeraRows = 64;
template <bool BF>
__global__ __launch_bounds__(256) void dora_vera_dd_part(const void* gBe, const void* Bsh,
                                                         const void* b, float* part, int64_t d_out,
                                                         int64_t r) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= r) return;
  const int64_t i0 = (int64_t)blockIdx.y * kVeraRows;
  const int64_t i1 = i0 + kVeraRows < d_out ? i0 + kVeraRows : d_out;
  float acc = 0.f;
  for (int64_t i = i0; i < i1; ++i)
    acc += Vec<BF>::scalar(gBe, i * r + j) * Vec<BF>::scalar(Bsh, i * r + j) *
           Vec<BF>::scalar(b, i);
  part[blockIdx.y * r + j] = acc;
}

// dd, stage 2: the row-block partial sums of each column, in order.
template <bool BF>
__global__ __launch_bounds__(256) void dora_vera_dd_final(const float* part, int64_t blocks,
                                                          void* dd, int64_t r) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= r) return;
  float acc = 0.f;
  for (int64_t z = 0; z < blocks; ++z) acc += part[z * r + j];
  if (BF)
    reinterpret_cast<uint16_t*>(dd)[j] = f32_to_bf16(acc);
  else
    reinterpret_cast<float*>(dd)[j] = acc;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int64_t vera_dd_blocks(int64_t d_out) { return cdiv(d_out, kVeraRows); }

hipError_t vera_scale(const void* Bsh, const void* b, const void* d, void* Be, int64_t d_out,
                      int64_t r, int dtype, hipStream_t st) {
  const int64_t n = d_out * r;
  if (n <= 0) return hipSuccess;
  LaunchTimer t("vera_scale", st);
  const dim3 grid((unsigned)cdiv(n, 256));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_vera_scale<true>, grid, dim3(256), 0, st, Bsh, b, d, Be, n, r);
  else
    hipLaunchKernelGGL(dora_vera_scale<false>, grid, dim3(256), 0, st, Bsh, b, d, Be, n, r);
  return hipGetLastError();
}

hipError_t vera_grads(const void* gBe, const void* Bsh, const void* b, const void* d, void* db,
                      void* dd, float* part, int64_t d_out, int64_t r, int dtype,
                      hipStream_t st) {
  const bool bf = dtype == kBF16;
  if (db && d_out > 0) {
    LaunchTimer t("vera_db", st);
    const dim3 grid((unsigned)cdiv(d_out, 4));
    if (bf)
      hipLaunchKernelGGL(dora_vera_db<true>, grid, dim3(256), 0, st, gBe, Bsh, d, db, d_out, r);
    else
      hipLaunchKernelGGL(dora_vera_db<false>, grid, dim3(256), 0, st, gBe, Bsh, d, db, d_out, r);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (dd && r > 0) {
    LaunchTimer t("vera_dd", st);
    const int64_t blocks = vera_dd_blocks(d_out);
    if (blocks > 0) {
      const dim3 g1((unsigned)cdiv(r, 256), (unsigned)blocks);
      if (bf)
        hipLaunchKernelGGL(dora_vera_dd_part<true>, g1, dim3(256), 0, st, gBe, Bsh, b, part, d_out, r);
      else
        hipLaunchKernelGGL(dora_vera_dd_part<false>, g1, dim3(256), 0, st, gBe, Bsh, b, part, d_out, r);
    }
    const dim3 g2((unsigned)cdiv(r, 256));
    if (bf)
      hipLaunchKernelGGL(dora_vera_dd_final<true>, g2, dim3(256), 0, st, part, blocks, dd, r);
    else
      hipLaunchKernelGGL(dora_vera_dd_final<false>, g2, dim3(256), 0, st, part, blocks, dd, r);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t gram_finalize(const float* part, int splits, int64_t r, float scale, int dtype,
                         void* g_hi, void* g_lo, hipStream_t st, const char* label) {
  if (r <= 0) return hipSuccess;
  LaunchTimer t(label, st);
  hipLaunchKernelGGL(dora_gram_finalize, dim3((unsigned)cdiv(r * r, 256)), dim3(256), 0, st, part,
                     splits, r * r, scale, dtype == kBF16 ? 1 : 0, g_hi, g_lo);
  return hipGetLastError();
}

hipError_t exact_prep(const void* m, const float* norm, const float* dm, const void* B, float s,
                      float* kappa, void* Bk, int64_t d_out, int64_t r, int dtype,
                      hipStream_t st) {
  LaunchTimer t("exact_prep", st);
  const dim3 grid((unsigned)cdiv(d_out * (r > 0 ? r : 1), 256));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_exact_prep<true>, grid, dim3(256), 0, st, m, norm, dm, B, s, kappa, Bk,
                       d_out, r);
  else
    hipLaunchKernelGGL(dora_exact_prep<false>, grid, dim3(256), 0, st, m, norm, dm, B, s, kappa,
                       Bk, d_out, r);
  return hipGetLastError();
}

hipError_t db_combine(const float* d1, int d1_splits, const float* q, int q_splits,
                      const float* kappa, void* dB, int64_t d_out, int64_t r, int dtype,
                      hipStream_t st) {
  LaunchTimer t("dB_combine", st);
  const int64_t n = d_out * r;
  const dim3 grid((unsigned)cdiv(n, 256));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_db_combine<true>, grid, dim3(256), 0, st, d1, d1_splits, q, q_splits,
                       kappa, dB, n, r);
  else
    hipLaunchKernelGGL(dora_db_combine<false>, grid, dim3(256), 0, st, d1, d1_splits, q, q_splits,
                       kappa, dB, n, r);
  return hipGetLastError();
}

hipError_t row_norm(const void* W0, const void* B, const float* P, int p_splits, float* norm,
                    int64_t d_out, int64_t d_in, int64_t r, int dtype, hipStream_t st) {
  LaunchTimer t("row_norm", st);
  const dim3 grid((unsigned)cdiv(d_out, 4));
  const int64_t stride = d_out * r;
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_row_norm<true>, grid, dim3(256), 0, st, W0, B, P, p_splits, stride,
                       norm, d_out, d_in, r);
  else
    hipLaunchKernelGGL(dora_row_norm<false>, grid, dim3(256), 0, st, W0, B, P, p_splits, stride,
                       norm, d_out, d_in, r);
  return hipGetLastError();
}

hipError_t compose_fwd(void* y, const void* slora, const void* m, const float* norm, int64_t T,
                       int64_t d_out, int dtype, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  LaunchTimer t("compose_fwd", st);
  const int64_t vec = dtype == kBF16 ? 8 : 4;
  const int64_t tpb = 16;
  const dim3 grid((unsigned)cdiv(d_out / vec, 256), (unsigned)cdiv(T, tpb));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_compose_fwd<true>, grid, dim3(256), 0, st, y, slora, m, norm, T, d_out,
                       tpb);
  else
    hipLaunchKernelGGL(dora_compose_fwd<false>, grid, dim3(256), 0, st, y, slora, m, norm, T,
                       d_out, tpb);
  return hipGetLastError();
}

hipError_t compose_bwd(const void* gy, const void* y, const void* m, const float* norm, void* gz,
                       float* dm_part, int64_t T, int64_t d_out, int64_t tokens_per_block,
                       int dtype, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  LaunchTimer t("compose_bwd", st);
  const int64_t vec = dtype == kBF16 ? 8 : 4;
  const dim3 grid((unsigned)cdiv(d_out / vec, 256), (unsigned)cdiv(T, tokens_per_block));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_compose_bwd<true>, grid, dim3(256), 0, st, gy, y, m, norm, gz, dm_part,
                       T, d_out, tokens_per_block);
  else
    hipLaunchKernelGGL(dora_compose_bwd<false>, grid, dim3(256), 0, st, gy, y, m, norm, gz,
                       dm_part, T, d_out, tokens_per_block);
  return hipGetLastError();
}

hipError_t scale_b_rows_t(const void* B, const void* m, const float* norm, float s, void* Bgt,
                          int64_t d_out, int64_t r, int dtype, hipStream_t st) {
  if (d_out <= 0 || r <= 0) return hipSuccess;
  LaunchTimer t("bg_scale", st);
  const dim3 grid((unsigned)cdiv(d_out, kTb), (unsigned)cdiv(r, kTb));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_scale_b_rows_t<true>, grid, dim3(256), 0, st, B, m, norm, s, Bgt,
                       d_out, r);
  else
    hipLaunchKernelGGL(dora_scale_b_rows_t<false>, grid, dim3(256), 0, st, B, m, norm, s, Bgt,
                       d_out, r);
  return hipGetLastError();
}

hipError_t dm_finalize(const float* dm_part, int64_t blocks, const void* m, float* dm,
                       int64_t d_out, const DmRecompute& z, int dtype, hipStream_t st) {
  LaunchTimer t("dm_finalize", st);
  const dim3 grid((unsigned)cdiv(d_out, 64));
  if (dtype == kBF16)
    hipLaunchKernelGGL(dora_dm_finalize<true>, grid, dim3(256), 0, st, dm_part, blocks, m, dm,
                       d_out, z.norm, z.gy, z.x, z.W0, z.A, z.B, z.s, z.T, z.d_in, z.r);
  else
    hipLaunchKernelGGL(dora_dm_finalize<false>, grid, dim3(256), 0, st, dm_part, blocks, m, dm,
                       d_out, z.norm, z.gy, z.x, z.W0, z.A, z.B, z.s, z.T, z.d_in, z.r);
  return hipGetLastError();
}

}  // namespace dora
