// One-token decode steps, gfx950: the recurrent mode the Mamba skill page
// ("Dual Computation Modes") uses for generation.  Both kernels read and update
// a small per-row state in place and touch every state element once, so they
// are bound by memory latency at these sizes.
//
// conv:  out = SiLU(bias + w[:,0] x_{t-3} + w[:,1] x_{t-2} + w[:,2] x_{t-1} + w[:,3] x_t),
//        then the window (x_{t-3}, x_{t-2}, x_{t-1}) <- (x_{t-2}, x_{t-1}, x_t);
//        a reset (document start at this token) clears the window first.
// scan:  dt = softplus(delta + delta_bias);  h <- exp(dt A) h + dt u B  (h <- 0
//        first on a reset);  out = (C . h + D u) silu(z).
// Both in one launch: the scan step forms u with the conv step's arithmetic.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void conv1d_update_kernel(const void* __restrict__ x, void* __restrict__ conv_state,
                                                            const float* __restrict__ weight,
                                                            const float* __restrict__ bias,
                                                            const uint8_t* __restrict__ reset, void* __restrict__ out,
                                                            int64_t batch, int64_t dim, bool apply_silu) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= batch * dim) return;
    const int64_t b = i / dim, d = i % dim;
    const bool clear = reset != nullptr && reset[b] != 0;
    float s[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) s[k] = clear ? 0.0f : Elem<T>::load(conv_state, i * 3 + k);
    const float xt = Elem<T>::load(x, i);
    const float* w = weight + d * 4;
    float acc = bias != nullptr ? bias[d] : 0.0f;
    acc = __builtin_fmaf(w[0], s[0], acc);
    acc = __builtin_fmaf(w[1], s[1], acc);
    acc = __builtin_fmaf(w[2], s[2], acc);
    acc = __builtin_fmaf(w[3], xt, acc);
    Elem<T>::store(out, i, apply_silu ? silu_f(acc) : acc);
    Elem<T>::store(conv_state, i * 3 + 0, s[1]);
    Elem<T>::store(conv_state, i * 3 + 1, s[2]);
    Elem<T>::store(conv_state, i * 3 + 2, xt);
}

// G = NT / 4 consecutive lanes own one (row, channel): four states each, so the
// state row of a channel is read and written as contiguous 16-byte pieces and
// C . h is a sum over the G lanes (xor shuffles inside the group).  NT is the
// power of two at or above N; for N < NT the state rows are N long and each
// lane touches only its states below N, element by element.
// CONV: the conv step runs first in the same launch; every lane of the group
// forms u from the window (rounded to T, as the separate conv step stores it)
// and the group's first lane writes the window back.
template <typename T, int G, bool HEADS, bool CONV>
__global__ __launch_bounds__(256) void state_update_kernel(const StateUpdateArgs a) {
    const int N = static_cast<int>(a.dstate);
    const bool exact = N == 4 * G;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t chan = gid / G;                   // b * dim + d
    const int q = static_cast<int>(gid % G);        // which four states
    const bool live = chan < a.batch * a.dim;
    const int64_t cc = live ? chan : 0;             // inactive lanes still join the shuffles
    const int64_t b = cc / a.dim, d = cc % a.dim;
    const int64_t head = HEADS ? d / (a.dim / a.nheads) : 0;
    const int64_t nd = HEADS ? a.nheads : a.dim;
    const int64_t dsel = HEADS ? head : d;

    float dt = Elem<T>::load(a.delta, b * nd + dsel) + (a.delta_bias != nullptr ? a.delta_bias[dsel] : 0.0f);
    if (a.softplus) dt = softplus_f(dt);
    const bool clear = a.reset != nullptr && a.reset[b] != 0;
    float u;
    if constexpr (CONV) {
        float s[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) s[k] = clear ? 0.0f : Elem<T>::load(a.conv_state, cc * 3 + k);
        const float xt = Elem<T>::load(a.conv_x, cc);
        const float* cw = a.conv_w + d * 4;
        float acc = a.conv_b != nullptr ? a.conv_b[d] : 0.0f;
        acc = __builtin_fmaf(cw[0], s[0], acc);
        acc = __builtin_fmaf(cw[1], s[1], acc);
        acc = __builtin_fmaf(cw[2], s[2], acc);
        acc = __builtin_fmaf(cw[3], xt, acc);
        u = silu_f(acc);
        if constexpr (sizeof(T) == 2) u = bf16_to_f32(f32_to_bf16(u));
        if (live && q == 0) {
            Elem<T>::store(a.conv_state, cc * 3 + 0, s[1]);
            Elem<T>::store(a.conv_state, cc * 3 + 1, s[2]);
            Elem<T>::store(a.conv_state, cc * 3 + 2, xt);
            if (a.u_out != nullptr) Elem<T>::store(a.u_out, cc, u);
        }
    } else {
        u = Elem<T>::load(a.u, cc);
    }
    const float w = dt * u;

    float hv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (!clear) {
        if (exact) {
            const float4 h = reinterpret_cast<const float4*>(a.state)[cc * G + q];
            hv[0] = h.x; hv[1] = h.y; hv[2] = h.z; hv[3] = h.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * q + j < N) hv[j] = a.state[cc * N + 4 * q + j];
        }
    }
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = 4 * q + j;
        if (!exact && n >= N) continue;           // a padded state: stays zero, adds nothing
        const float Al = HEADS ? a.A[head] : a.A[d * N + n];
        const float decay = exp2_fast(dt * Al * kLog2e);
        hv[j] = __builtin_fmaf(decay, hv[j], w * Elem<T>::load(a.B, b * N + n));
        y = __builtin_fmaf(Elem<T>::load(a.C, b * N + n), hv[j], y);
    }
#pragma unroll
    for (int m = G / 2; m > 0; m >>= 1) y += __shfl_xor(y, m);
    if (!live) return;
    if (exact) {
        reinterpret_cast<float4*>(a.state)[cc * G + q] = make_float4(hv[0], hv[1], hv[2], hv[3]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * q + j < N) a.state[cc * N + 4 * q + j] = hv[j];
    }
    if (q == 0) {
        y = __builtin_fmaf(a.D != nullptr ? a.D[d] : 0.0f, u, y);
        if (a.z != nullptr) y *= silu_f(Elem<T>::load(a.z, cc));
        Elem<T>::store(a.out, cc, y);
    }
}

template <typename T, bool HEADS, bool CONV>
hipError_t launch_state_update_typed(const StateUpdateArgs& a) {
    int G = 1;
    while (4 * G < a.dstate) G *= 2;
    const int64_t threads = a.batch * a.dim * G;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    switch (G) {
        case 1: hipLaunchKernelGGL((state_update_kernel<T, 1, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        case 2: hipLaunchKernelGGL((state_update_kernel<T, 2, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        case 4: hipLaunchKernelGGL((state_update_kernel<T, 4, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        case 8: hipLaunchKernelGGL((state_update_kernel<T, 8, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        case 16: hipLaunchKernelGGL((state_update_kernel<T, 16, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        case 32: hipLaunchKernelGGL((state_update_kernel<T, 32, HEADS, CONV>), grid, dim3(256), 0, a.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool HEADS>
hipError_t launch_state_update_conv(const StateUpdateArgs& a) {
    return a.conv_x != nullptr ? launch_state_update_typed<T, HEADS, true>(a) : launch_state_update_typed<T, HEADS, false>(a);
}

}  // namespace

bool state_update_supported(int64_t dstate) { return dstate >= 1 && dstate <= 128; }

hipError_t launch_state_update(const StateUpdateArgs& a) {
    if (a.bf16) return a.nheads ? launch_state_update_conv<bf16_t, true>(a) : launch_state_update_conv<bf16_t, false>(a);
    return a.nheads ? launch_state_update_conv<float, true>(a) : launch_state_update_conv<float, false>(a);
}

hipError_t launch_conv1d_update(const ConvUpdateArgs& a) {
    const dim3 grid(static_cast<unsigned>((a.batch * a.dim + 255) / 256));
    if (a.bf16)
        hipLaunchKernelGGL(conv1d_update_kernel<bf16_t>, grid, dim3(256), 0, a.stream, a.x, a.conv_state, a.weight,
                           a.bias, a.reset, a.out, a.batch, a.dim, a.apply_silu);
    else
        hipLaunchKernelGGL(conv1d_update_kernel<float>, grid, dim3(256), 0, a.stream, a.x, a.conv_state, a.weight,
                           a.bias, a.reset, a.out, a.batch, a.dim, a.apply_silu);
    return hipGetLastError();
}

}  // namespace mamba
