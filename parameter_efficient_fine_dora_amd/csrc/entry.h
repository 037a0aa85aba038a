// Internal entry points shared by the C ABI's source files.
#pragma once
#include <stddef.h>

#include "../../include/dora.h"

namespace dora {

// dora_forward's body.  allow_side_stream = false keeps every launch on the
// caller's stream (no side stream or events are created).
int forward_impl(const dora_shape* shape, const void* x, const void* W0, const void* A,
                 const void* B, const void* m, void* y, float* norm_out, void* xs_out, void* ws,
                 size_t ws_bytes, void* hip_stream, bool allow_side_stream);

}  // namespace dora
