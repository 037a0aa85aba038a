// Measurement probes: the dense bf16 MFMA rate and the streaming HBM rate
// this chip sustains, against which the kernels are reported beside the
// published peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/dora.h"
#include "common.h"

namespace {

using dora::bf16x8;
using dora::f32x16;

// Independent accumulation chains per wave: enough to cover the MFMA latency,
// so the matrix pipe issues back to back.
constexpr int kChains = 4;

// Every wave runs kChains chains of v_mfma_f32_32x32x16_bf16 on register
// operands for `iters` steps; memory is touched only by the checksum store.
__global__ __launch_bounds__(256) void dora_mfma_probe(int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    a[q] = (__bf16)(0.125f * (float)((lane + q) & 7));
    b[q] = (__bf16)(0.0625f * (float)((lane * 3 + q) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// c = a + b over n float4 vectors (two streams in, one out: the access
// pattern of the compose kernels).  Workgroup w owns the contiguous vectors
// [1024 w, 1024 (w + 1)); each thread loads four of them, 256 apart, before
// its first store (this shape measured faster than a grid-stride loop).
__global__ __launch_bounds__(256) void dora_stream_probe(const float4* a, const float4* b,
                                                          float4* c, int64_t n) {
  constexpr int U = 4;
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  float4 x[U], y[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * 256;
    if (i < n) {
      x[u] = a[i];
      y[u] = b[i];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * 256;
    if (i < n)
      c[i] = make_float4(x[u].x + y[u].x, x[u].y + y[u].y, x[u].z + y[u].z, x[u].w + y[u].w);
  }
}

}  // namespace

DORA_API int dora_probe_stream(const void* a, const void* b, void* c, int64_t bytes,
                               void* hip_stream) {
  if (!a || !b || !c) return DORA_ERR_NULL;
  if (bytes < 16 || bytes % 16) return DORA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
       reinterpret_cast<uintptr_t>(c)) & 15u)
    return DORA_ERR_ALIGN;
  const int64_t n = bytes / 16;
  const int64_t blocks = (n + 1023) / 1024;
  if (blocks > 0x7fffffff) return DORA_ERR_SHAPE;
  hipLaunchKernelGGL(dora_stream_probe, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(hip_stream), reinterpret_cast<const float4*>(a),
                     reinterpret_cast<const float4*>(b), reinterpret_cast<float4*>(c), n);
  return hipGetLastError() == hipSuccess ? DORA_OK : DORA_ERR_HIP;
}

DORA_API int dora_probe_mfma(int64_t iters, int blocks, float* out, void* hip_stream) {
  if (iters < 1 || blocks < 1 || !out) return DORA_ERR_SHAPE;
  hipLaunchKernelGGL(dora_mfma_probe, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(hip_stream), iters, out);
  return hipGetLastError() == hipSuccess ? DORA_OK : DORA_ERR_HIP;
}

DORA_API double dora_probe_mfma_flops(int64_t iters, int blocks) {
  return (double)blocks * 4.0 * (double)iters * kChains * 2.0 * 32.0 * 32.0 * 16.0;
}
