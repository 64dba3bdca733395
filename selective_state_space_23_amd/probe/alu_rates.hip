// Issue-rate probe of the gfx950 vector ALU: how many wave64 instructions of a
// kind one SIMD retires per shader clock, and the dependent latency of each.
//
// The selective scan's per-(t, d, n) work is one v_exp_f32 and a few fp32
// FMAs/multiplies, so its ALU floor depends on the transcendental rate relative
// to the FMA rate and on whether the two overlap.  Each kernel below runs
// independent chains of one instruction kind (or a fixed mix of kinds) in every
// lane; the host times it with HIP events and reads the shader clock from
// s_memtime against the constant 100 MHz s_memrealtime in every workgroup.
//
// Kinds: 0 v_fma_f32, 1 v_mul_f32, 2 v_add_f32, 3 v_exp_f32, 4 v_log_f32,
// 5 v_rcp_f32, 6 one v_exp_f32 per FMA, 7 one v_exp_f32 per 3 FMAs,
// 8 one v_exp_f32 per 5 FMAs (the mixes use independent chains, so an exp and
// an FMA can overlap if the hardware allows it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace {

constexpr int kThreads = 256;

template <int KIND>
__device__ __forceinline__ float op(float x, float a, float b) {
    if constexpr (KIND == 0) return __builtin_fmaf(x, a, b);
    if constexpr (KIND == 1) return x * a;
    if constexpr (KIND == 2) return x + a;
    if constexpr (KIND == 3) return __builtin_amdgcn_exp2f(-x);
    if constexpr (KIND == 4) return __builtin_amdgcn_logf(__builtin_fabsf(x));
    if constexpr (KIND == 5) return __builtin_amdgcn_rcpf(x);
    return x;
}

// Instruction mix of one unrolled step: E exponentials and F FMAs on E + F
// independent chains (E + F = 8 for the throughput kernels).
template <int KIND> struct Mix;
template <> struct Mix<6> { static constexpr int E = 4, F = 4; };
template <> struct Mix<7> { static constexpr int E = 2, F = 6; };
template <> struct Mix<8> { static constexpr int E = 1, F = 5; };

// CHAINS independent chains per lane, 8 steps unrolled per loop trip.
template <int KIND, int CHAINS>
__global__ __launch_bounds__(kThreads) void rate_kernel(float* out, unsigned long long* clk, int iters, float a,
                                                        float b) {
    float x[CHAINS];
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) x[i] = 0.5f + 0.001f * static_cast<float>(threadIdx.x + i);
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if constexpr (KIND <= 5) {
#pragma unroll
                for (int i = 0; i < CHAINS; ++i) x[i] = op<KIND>(x[i], a, b);
            } else {
                constexpr int E = Mix<KIND>::E, F = Mix<KIND>::F;
#pragma unroll
                for (int i = 0; i < E; ++i) x[i] = op<3>(x[i], a, b);
#pragma unroll
                for (int i = E; i < E + F; ++i) x[i] = op<0>(x[i], a, b);
            }
        }
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) acc += x[i];
    out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

template <int KIND, int CHAINS>
hipError_t launch(int blocks, int threads, int iters, float* out, unsigned long long* clk, hipStream_t s) {
    hipLaunchKernelGGL((rate_kernel<KIND, CHAINS>), dim3(blocks), dim3(threads), 0, s, out, clk, iters, 0.999f,
                       1e-3f);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(int chains, int blocks, int threads, int iters, float* out, unsigned long long* clk,
                       hipStream_t s) {
    if constexpr (KIND >= 6) {
        if (chains != Mix<KIND>::E + Mix<KIND>::F) return hipErrorInvalidValue;
        return launch<KIND, Mix<KIND>::E + Mix<KIND>::F>(blocks, threads, iters, out, clk, s);
    } else {
        if (chains == 1) return launch<KIND, 1>(blocks, threads, iters, out, clk, s);
        if (chains == 8) return launch<KIND, 8>(blocks, threads, iters, out, clk, s);
        return hipErrorInvalidValue;
    }
}

// The library's own device softplus (device_common.hpp) on given inputs, so that
// a test can check its accuracy against a float64 reference.
__global__ void softplus_kernel(const float* v, float* out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = mamba::softplus_f(v[i]);
}

}  // namespace

extern "C" {

// out[i] = softplus of v[i] as the library's kernels evaluate it.  Returns a
// hipError_t value.
int probe_softplus(const float* v, float* out, int n, void* stream) {
    if (n < 0 || (n > 0 && (!v || !out))) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(softplus_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), v,
                       out, n);
    return hipGetLastError();
}

// One timed launch.  kind: 0..8 as above; chains: 1 (dependent latency) or 8
// (throughput; the mixes 6..8 take E + F chains: 8, 8, 6).  out holds
// blocks * threads floats, clk 2 * blocks 64-bit words (per workgroup: shader
// clocks, 100 MHz ticks).  threads <= 256.  Returns a hipError_t value.
int probe_alu_rate(int kind, int chains, int blocks, int threads, int iters, float* out,
                   unsigned long long* clk, void* stream) {
    if (threads < 1 || threads > kThreads || blocks < 1 || iters < 1 || !out || !clk) return hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
        case 0: return launch_kind<0>(chains, blocks, threads, iters, out, clk, s);
        case 1: return launch_kind<1>(chains, blocks, threads, iters, out, clk, s);
        case 2: return launch_kind<2>(chains, blocks, threads, iters, out, clk, s);
        case 3: return launch_kind<3>(chains, blocks, threads, iters, out, clk, s);
        case 4: return launch_kind<4>(chains, blocks, threads, iters, out, clk, s);
        case 5: return launch_kind<5>(chains, blocks, threads, iters, out, clk, s);
        case 6: return launch_kind<6>(chains, blocks, threads, iters, out, clk, s);
        case 7: return launch_kind<7>(chains, blocks, threads, iters, out, clk, s);
        case 8: return launch_kind<8>(chains, blocks, threads, iters, out, clk, s);
        default: return hipErrorInvalidValue;
    }
}

}  // extern "C"
