// Outputs of calls that have no tokens: a final state equal to the initial one,
// gradient sums over no tokens equal to zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

// dst[i] = src ? src[i] : 0 for i < n (a kernel, not a memset: the call may sit
// inside a captured graph).
hipError_t launch_fill(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace mamba
