// The whole forward of a small float32 DoRA layer in two kernels (Scaling DoRA
// summary page, English abstract: the factored norm and the single-pass
// compose; DoRA reading notes, Alg. 1).  Layers this small are all
// launch latency on the multi-kernel path.  Here one pass over K = d_in
// accumulates, for each block of 16 output rows,
//   xs = x A^T (before the scale by s), z_t,i = x_t . W0_i,
//   G = A A^T (r x r), U_i = W0_i A^T and ||W0_i||^2,
// with K split over workgroups where the row blocks alone cannot fill the chip;
// a second kernel sums the splits in order and forms
//   n_i = sqrt(max(0, ||W0_i||^2 + 2s B_i . U_i + s^2 B_i G B_i^T)),
//   y_t,i = z'_t,i + (g_i - 1) z'_t,i with z' = z + xs_t . B_i, g_i - 1 = (m_i - n_i) / n_i.
// Every workgroup forms G and x A^T over its K range (small next to its rows'
// work); those of row block 0 store them.  All sums are float32 in a fixed order.
#include "common.h"
#include "kernels.h"

namespace dora {
namespace {

constexpr int kSmRows = 16;   // output rows per workgroup
constexpr int kSmK = 64;      // K chunk
constexpr int kSmPad = kSmK + 1;
constexpr int kSmCols = kSmallMaxRank + kSmRows;   // rows of [A ; W0 block] in a chunk (48)
// 256 threads as 16 x 16: 4 tokens x 3 columns of X and 3 x 3 of Q each.
static_assert(16 * 4 == kSmallMaxTokens && 16 * 3 == kSmCols, "register tiles cover X and Q");
static_assert((kSmCols * kSmK) % 256 == 0 && (kSmallMaxTokens * kSmK) % 256 == 0,
              "chunk loads divide evenly over 256 threads");
// partial-sum layout (float32), matching small_forward_plan
constexpr int kZPart = kSmallMaxTokens * kSmRows;             // z [64][16]
constexpr int kUPart = kSmRows * (kSmallMaxRank + 1);         // U | ||W0_i||^2 [16][33]
constexpr int kRowPart = kZPart + kUPart;
constexpr int kXPart = kSmallMaxTokens * kSmallMaxRank;       // x A^T [64][32]
constexpr int kGPart = kSmallMaxRank * kSmallMaxRank;         // A A^T [32][32]
constexpr int kSplitPart = kXPart + kGPart;

// Grid (row blocks, K splits).  Per 64-deep chunk the workgroup stages x
// [T x 64] and [A ; W0 block] [(r + 16) x 64] in LDS and accumulates, with
// 4 x 3 and 3 x 3 register tiles per thread (each LDS value feeds three or
// four FMAs):
//   X = x [A ; W0 block]^T      (x A^T and z)
//   Q = [A ; W0 block] [A ; W0 block]^T   (G, U and ||W0_i||^2 on its diagonal)
__global__ __launch_bounds__(256) void dora_small_partials(
    const float* __restrict__ x, const float* __restrict__ W0, const float* __restrict__ A,
    float* __restrict__ part, int T, int d_out, int d_in, int r, int chunks) {
  __shared__ float sX[kSmallMaxTokens][kSmPad];
  __shared__ float sR[kSmCols][kSmPad];                   // [A ; W0 block] chunk
  __shared__ float sQ[kSmCols][kSmCols + 1];
  __shared__ float sXR[kSmallMaxTokens][kSmCols + 1];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x, kc = blockIdx.y, nrb = gridDim.x;
  const int i0 = rb * kSmRows;
  const int k_begin = kc * chunks * kSmK, k_end = min(d_in, k_begin + chunks * kSmK);
  const int tg = tid / 16, cg = tid % 16;   // X tile: tokens 4tg.., columns 3cg..
  const int qa = tg, qb = cg;               // Q tile: rows 3qa.., columns 3qb..
  float aX[4][3], aQ[3][3];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 3; ++v) aX[u][v] = 0.f;
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int v = 0; v < 3; ++v) aQ[u][v] = 0.f;

  // The next chunk's global loads are issued before the current chunk's FMAs
  // (held in registers), so their latency hides behind the arithmetic.
  constexpr int kRLoads = kSmCols * kSmK / 256;           // 12
  constexpr int kXLoads = kSmallMaxTokens * kSmK / 256;   // 16
  float pr[kRLoads], px[kXLoads];
  auto fetch = [&](int k0) {
    const int kw = min(kSmK, k_end - k0);
#pragma unroll
    for (int j = 0; j < kRLoads; ++j) {
      const int e = tid + 256 * j, row = e / kSmK, kk = e % kSmK;
      float v = 0.f;
      if (kk < kw) {
        if (row < r) {
          v = A[(int64_t)row * d_in + k0 + kk];
        } else if (row >= kSmallMaxRank) {
          const int i = i0 + row - kSmallMaxRank;
          if (i < d_out) v = W0[(int64_t)i * d_in + k0 + kk];
        }
      }
      pr[j] = v;
    }
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int e = tid + 256 * j, t = e / kSmK, kk = e % kSmK;
      px[j] = (t < T && kk < kw) ? x[(int64_t)t * d_in + k0 + kk] : 0.f;
    }
  };
  fetch(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += kSmK) {
    // rows 0..r-1 of sR: A; rows kSmallMaxRank.. : the W0 block; the rest zero
#pragma unroll
    for (int j = 0; j < kRLoads; ++j) {
      const int e = tid + 256 * j;
      sR[e / kSmK][e % kSmK] = pr[j];
    }
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int e = tid + 256 * j;
      sX[e / kSmK][e % kSmK] = px[j];
    }
    __syncthreads();
    if (k0 + kSmK < k_end) fetch(k0 + kSmK);
    for (int kk = 0; kk < kSmK; ++kk) {
      float xv[4], rv[3], qv[3], pv[3];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[u] = sX[4 * tg + u][kk];
#pragma unroll
      for (int v = 0; v < 3; ++v) {
        rv[v] = sR[3 * cg + v][kk];
        qv[v] = sR[3 * qa + v][kk];
        pv[v] = sR[3 * qb + v][kk];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 3; ++v) aX[u][v] = fmaf(xv[u], rv[v], aX[u][v]);
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int v = 0; v < 3; ++v) aQ[u][v] = fmaf(qv[u], pv[v], aQ[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 3; ++v) sXR[4 * tg + u][3 * cg + v] = aX[u][v];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int v = 0; v < 3; ++v) sQ[3 * qa + u][3 * qb + v] = aQ[u][v];
  __syncthreads();

  float* rp = part + ((int64_t)kc * nrb + rb) * kRowPart;
  for (int e = tid; e < kZPart; e += 256) rp[e] = sXR[e / kSmRows][kSmallMaxRank + e % kSmRows];
  for (int e = tid; e < kUPart; e += 256) {
    const int il = e / (kSmallMaxRank + 1), c = e % (kSmallMaxRank + 1);
    rp[kZPart + e] = sQ[kSmallMaxRank + il][c < kSmallMaxRank ? c : kSmallMaxRank + il];
  }
  if (rb == 0) {
    float* sp = part + (int64_t)gridDim.y * nrb * kRowPart + (int64_t)kc * kSplitPart;
    for (int e = tid; e < kXPart; e += 256) sp[e] = sXR[e / kSmallMaxRank][e % kSmallMaxRank];
    for (int e = tid; e < kGPart; e += 256) sp[kXPart + e] = sQ[e / kSmallMaxRank][e % kSmallMaxRank];
  }
}

// Grid (row blocks), 1024 threads: the split sums in split order, then the
// norm and compose.  The partials a thread sums are loaded together before
// any is added, so the kernel waits on memory about once, not once per split.
constexpr int kFinThreads = 1024;
constexpr int kFinElems = kRowPart + kSplitPart;                          // 4624
constexpr int kFinPerThread = (kFinElems + kFinThreads - 1) / kFinThreads;   // 5
constexpr int kMaxSplits = (int)((kSmallMaxDin + kSmK - 1) / kSmK);         // 16

__global__ __launch_bounds__(kFinThreads) void dora_small_finish(
    const float* __restrict__ part, const float* __restrict__ B, const float* __restrict__ m,
    float s, float* __restrict__ y, float* __restrict__ norm, float* __restrict__ xs_out, int T,
    int d_out, int r, int ksplits) {
  __shared__ float sZ[kSmallMaxTokens][kSmRows + 1];
  __shared__ float sU[kSmRows][kSmallMaxRank + 1];
  __shared__ float sXs[kSmallMaxTokens][kSmallMaxRank + 1];
  __shared__ float sG[kSmallMaxRank][kSmallMaxRank + 1];
  __shared__ float sB[kSmRows][kSmallMaxRank + 1];
  __shared__ float sN[kSmRows];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x, nrb = gridDim.x, i0 = rb * kSmRows;
  // element e < kRowPart: this row block's z | U | ||W0_i||^2; else the
  // split's x A^T | A A^T (written by row block 0)
  const float* rp = part + (int64_t)rb * kRowPart;
  const float* sp = part + (int64_t)ksplits * nrb * kRowPart - kRowPart;
  const int64_t rstride = (int64_t)nrb * kRowPart;
  float v[kFinPerThread][kMaxSplits];
#pragma unroll
  for (int j = 0; j < kFinPerThread; ++j) {
    const int e = tid + kFinThreads * j;
    if (e < kFinElems) {
      const float* src = e < kRowPart ? rp + e : sp + e;
      const int64_t stride = e < kRowPart ? rstride : kSplitPart;
#pragma unroll
      for (int z = 0; z < kMaxSplits; ++z)
        if (z < ksplits) v[j][z] = src[z * stride];
    }
  }
#pragma unroll
  for (int j = 0; j < kFinPerThread; ++j) {
    const int e = tid + kFinThreads * j;
    if (e < kFinElems) {
      float a = 0.f;
#pragma unroll
      for (int z = 0; z < kMaxSplits; ++z)
        if (z < ksplits) a += v[j][z];
      if (e < kZPart) {
        sZ[e / kSmRows][e % kSmRows] = a;
      } else if (e < kRowPart) {
        const int u = e - kZPart;
        sU[u / (kSmallMaxRank + 1)][u % (kSmallMaxRank + 1)] = a;
      } else if (e < kRowPart + kXPart) {
        const int u = e - kRowPart;
        sXs[u / kSmallMaxRank][u % kSmallMaxRank] = s * a;   // xs = s (x A^T)
      } else {
        const int u = e - kRowPart - kXPart;
        sG[u / kSmallMaxRank][u % kSmallMaxRank] = a;
      }
    }
  }
  for (int e = tid; e < kSmRows * kSmallMaxRank; e += kFinThreads) {
    const int il = e / kSmallMaxRank, q = e % kSmallMaxRank, i = i0 + il;
    sB[il][q] = (i < d_out && q < r) ? B[(int64_t)i * r + q] : 0.f;
  }
  __syncthreads();

  // n_i = sqrt(max(0, ||W0_i||^2 + 2s B_i . U_i + s^2 B_i G B_i^T)), sixteen lanes per row
  if (tid < 16 * kSmRows) {   // whole waves, so the width-16 shuffles see full groups
    const int il = tid / 16, l = tid % 16, i = i0 + il;
    float cross = 0.f, gram = 0.f;
    for (int q = l; q < r; q += 16) {
      float tq = 0.f;
      for (int q2 = 0; q2 < r; ++q2) tq = fmaf(sG[q][q2], sB[il][q2], tq);
      cross = fmaf(sB[il][q], sU[il][q], cross);
      gram = fmaf(sB[il][q], tq, gram);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      cross += __shfl_xor(cross, off, 16);
      gram += __shfl_xor(gram, off, 16);
    }
    if (l == 0) {
      const float n2 = sU[il][kSmallMaxRank] + 2.f * s * cross + s * s * gram;
      const float n = sqrtf(fmaxf(n2, 0.f));
      sN[il] = n;
      if (i < d_out) norm[i] = n;
    }
  }
  if (rb == 0)
    for (int e = tid; e < T * r; e += kFinThreads) xs_out[e] = sXs[e / r][e % r];
  __syncthreads();

  // y = z' + (g - 1) z' with z' = x_t . W0_i + xs_t . B_i
  for (int e = tid; e < T * kSmRows; e += kFinThreads) {
    const int t = e / kSmRows, il = e % kSmRows, i = i0 + il;
    if (i < d_out) {
      float z = sZ[t][il];
      for (int q = 0; q < r; ++q) z = fmaf(sXs[t][q], sB[il][q], z);
      const float nv = fmaxf(sN[il], kNormEps);
      const float gm1 = (m[i] - nv) / nv;
      y[(int64_t)t * d_out + i] = z + gm1 * z;
    }
  }
}

}  // namespace

hipError_t small_forward(const float* x, const float* W0, const float* A, const float* B,
                         const float* m, float s, float* y, float* norm, float* xs, float* part,
                         int64_t T, int64_t d_out, int64_t d_in, int64_t r, hipStream_t st) {
  if (!small_forward_fits(T, d_out, d_in, r)) return hipErrorInvalidValue;
  const SmallPlan p = small_forward_plan(d_out, d_in);
  if (p.ksplits > kMaxSplits) return hipErrorInvalidValue;
  static_assert(kRowPart == 64 * 16 + 16 * 33 && kSplitPart == 64 * 32 + 32 * 32,
                "partial layout matches small_forward_plan");
  {
    LaunchTimer t("small_partials", st);
    hipLaunchKernelGGL(dora_small_partials, dim3((unsigned)p.row_blocks, (unsigned)p.ksplits),
                       dim3(256), 0, st, x, W0, A, part, (int)T, (int)d_out, (int)d_in, (int)r,
                       (int)p.chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchTimer t("small_finish", st);
  hipLaunchKernelGGL(dora_small_finish, dim3((unsigned)p.row_blocks), dim3(kFinThreads), 0, st, part, B,
                     m, s, y, norm, xs, (int)T, (int)d_out, (int)r, (int)p.ksplits);
  return hipGetLastError();
}

}  // namespace dora
