// dora_forward_noalloc: dora_forward for callers that cannot allocate device
// memory (code under stream capture, tight serving loops).  Its workspace is a
// file-scope device array instead of a caller-provided buffer; everything else
// (validation, kernels, results) is dora_forward's.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is handed
// to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dora.h"
#include "entry.h"

namespace {

constexpr size_t kScratchBytes = DORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the workspace layout aligns regions to 256 bytes");

// Every GPU the library runs on holds one copy until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, or nullptr if it cannot
// be had (the lookup runs once per device; a failed lookup is retried).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

DORA_API int dora_forward_noalloc(const dora_shape* shape, const void* x, const void* W0,
                                  const void* A, const void* B, const void* m, void* y,
                                  float* norm_out, void* xs_out, void* hip_stream) {
  if (!shape) return DORA_ERR_NULL;
  // too large for the static workspace (0 = invalid shape: dora_forward reports why)
  if (dora_workspace_bytes(shape, DORA_OP_FORWARD) > kScratchBytes) return DORA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return DORA_ERR_HIP;
  return dora::forward_impl(shape, x, W0, A, B, m, y, norm_out, xs_out, ws, kScratchBytes,
                            hip_stream, /*allow_side_stream=*/false);
}

}  // extern "C"
