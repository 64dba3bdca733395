// State-size padding for the scan kernels, gfx950.
//
// The chunked scan and its backward are compiled for a few state sizes N (4, 8,
// 16 per channel; 16, 32, 64, 128 for fp32 scalar-A heads; multiples of 8 for
// the bf16 heads matrix form).  Any other N runs on copies of B, C, A and the
// states padded with zeros to the next compiled size NT, placed in the caller's
// workspace: a padded state n >= N has A = 0 (decay 1), B = 0 (no input) and
// C = 0 (no output), so it stays zero and adds nothing to y; the results for
// n < N are exactly those of the unpadded recurrence.  Gradients are computed
// for the padded problem and the first N states of each row are copied out.
#include "launch.hpp"

namespace mamba {

namespace {

// dst[r, k] = src[r, k] for k < n, 0 for n <= k < nt; rows of esz-byte elements.
template <typename E>
__global__ __launch_bounds__(256) void pad_rows_kernel(const E* __restrict__ src, E* __restrict__ dst, int64_t rows,
                                                       int n, int nt) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= rows * nt) return;
    const int64_t r = i / nt;
    const int k = static_cast<int>(i % nt);
    dst[i] = k < n ? src[r * n + k] : E(0);
}

// dst[r, k] = src[r, k] for k < n (rows of nt elements in src, n in dst).
template <typename E>
__global__ __launch_bounds__(256) void unpad_rows_kernel(const E* __restrict__ src, E* __restrict__ dst, int64_t rows,
                                                         int n, int nt) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= rows * n) return;
    const int64_t r = i / n;
    const int k = static_cast<int>(i % n);
    dst[i] = src[r * nt + k];
}

dim3 grid_for(int64_t count) { return dim3(static_cast<unsigned>((count + 255) / 256)); }

}  // namespace

hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int n, int nt, int esz, hipStream_t stream) {
    if (rows * nt == 0) return hipSuccess;
    if (esz == 2)
        hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, grid_for(rows * nt), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, n, nt);
    else
        hipLaunchKernelGGL(pad_rows_kernel<uint32_t>, grid_for(rows * nt), dim3(256), 0, stream,
                           static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), rows, n, nt);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(const void* src, void* dst, int64_t rows, int n, int nt, int esz, hipStream_t stream) {
    if (rows * n == 0) return hipSuccess;
    if (esz == 2)
        hipLaunchKernelGGL(unpad_rows_kernel<uint16_t>, grid_for(rows * n), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, n, nt);
    else
        hipLaunchKernelGGL(unpad_rows_kernel<uint32_t>, grid_for(rows * n), dim3(256), 0, stream,
                           static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), rows, n, nt);
    return hipGetLastError();
}

}  // namespace mamba
