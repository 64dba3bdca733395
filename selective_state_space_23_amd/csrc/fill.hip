// Copy or zero-fill of a float32 array, for the outputs of calls with no tokens.
#include "fill.hpp"

namespace mamba {

namespace {

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                   int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = src != nullptr ? src[i] : 0.0f;
}

}  // namespace

hipError_t launch_fill(float* dst, const float* src, int64_t n, hipStream_t stream) {
    if (dst == nullptr || n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace mamba
