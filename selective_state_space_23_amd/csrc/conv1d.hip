// Depthwise causal conv1d (width 4) + SiLU over packed documents, gfx950.
//
// What it computes ("Mamba: Selective State Spaces (S6)" section of the Mamba
// skill page, with the axolotl page's per-document restart):
//     u[b,t,d] = act(bias[d] + sum_{j=0..3} w[d, 3-j] * x[b, t-j, d])
// where a tap whose token precedes the start of token t's document reads zero.
//
// Mapping.  The op is pure streaming (about 4 bytes in and out per element at
// bf16, ~15 VALU slots per element), so it is laid out for HBM:
//   - each thread owns VEC consecutive channels (16 bytes of x) and walks a tile
//     of TT consecutive tokens, so every load and store of a wave is one
//     contiguous 1 KiB span of the (B, L, D) row;
//   - the last three inputs live in a register shift register; a document start
//     (uniform across the block, known from a 64-bit ballot of the tile's
//     doc_start bytes) clears it, which zeroes exactly the taps that would cross
//     into the previous document;
//   - the three tokens before the tile are re-read as a halo (3/TT extra reads,
//     mostly L2 hits) and replayed through the same shift register.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

constexpr int kConvTile = 48;      // tokens per thread; kConvTile + 3 <= 64 for one ballot
constexpr int kConvBlock = 256;

template <typename T, int VEC, bool SILU>
__global__ __launch_bounds__(kConvBlock) void causal_conv1d_w4_kernel(
    const void* __restrict__ x, const float* __restrict__ weight, const float* __restrict__ bias,
    const uint8_t* __restrict__ doc_start, const void* __restrict__ conv_state, void* __restrict__ out,
    int64_t seqlen, int dim) {
    const int ngroups = (dim + VEC - 1) / VEC;   // VEC == 1 when dim % VEC != 0
    const int g = blockIdx.x * kConvBlock + threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvTile;
    const int64_t b = blockIdx.z;
    const int64_t row = b * seqlen;

    // Document starts of tokens t0-3 .. t0+kConvTile-1 as one wave-uniform mask:
    // bit i <-> token t0 - 3 + i.  Token 0 of the row starts a document unless the
    // row continues a given history (conv_state).
    const int lane = threadIdx.x & 63;
    const int64_t tl = t0 - 3 + lane;
    bool is_start = false;
    if (lane < kConvTile + 3 && tl >= 0 && tl < seqlen)
        is_start = (tl == 0 && conv_state == nullptr) || (doc_start != nullptr && doc_start[row + tl] != 0);
    const uint64_t starts = __ballot(is_start);
    if (g >= ngroups) return;

    const int d0 = g * VEC;
    float w0[VEC], w1[VEC], w2[VEC], w3[VEC], bs[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        const float* wr = weight + 4 * (d0 + i);
        w0[i] = wr[0]; w1[i] = wr[1]; w2[i] = wr[2]; w3[i] = wr[3];
        bs[i] = bias ? bias[d0 + i] : 0.0f;
    }

    // h1 = x[t-1], h2 = x[t-2], h3 = x[t-3] restricted to token t's document.
    float h1[VEC], h2[VEC], h3[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {            // replay the halo tokens t0-3 .. t0-1
        const int64_t t = t0 - 3 + k;
        float xv[VEC];
        if (t >= 0) {
            VecIO<T, VEC>::load(x, (row + t) * dim + d0, xv);
        } else if (conv_state != nullptr) {  // (B, D, 3): x_{-3}, x_{-2}, x_{-1} of each channel
#pragma unroll
            for (int i = 0; i < VEC; ++i) xv[i] = Elem<T>::load(conv_state, (b * dim + d0 + i) * 3 + (3 + t));
        } else {
            continue;
        }
        const bool reset = (starts >> k) & 1ull;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            h3[i] = reset ? 0.0f : h2[i];
            h2[i] = reset ? 0.0f : h1[i];
            h1[i] = xv[i];
        }
    }

    const int64_t tend = (t0 + kConvTile < seqlen) ? t0 + kConvTile : seqlen;
    for (int64_t t = t0; t < tend; ++t) {
        float xv[VEC];
        VecIO<T, VEC>::load(x, (row + t) * dim + d0, xv);
        if ((starts >> (t - t0 + 3)) & 1ull) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
        }
        float yv[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            float acc = __builtin_fmaf(w3[i], xv[i], bs[i]);
            acc = __builtin_fmaf(w2[i], h1[i], acc);
            acc = __builtin_fmaf(w1[i], h2[i], acc);
            acc = __builtin_fmaf(w0[i], h3[i], acc);
            yv[i] = SILU ? silu_f(acc) : acc;
            h3[i] = h2[i];
            h2[i] = h1[i];
            h1[i] = xv[i];
        }
        VecIO<T, VEC>::store(out, (row + t) * dim + d0, yv);
    }
}

template <typename T, int VEC>
hipError_t launch_conv_vec(const ConvArgs& a) {
    const int ngroups = static_cast<int>((a.dim + VEC - 1) / VEC);
    dim3 grid((ngroups + kConvBlock - 1) / kConvBlock,
              static_cast<unsigned>((a.seqlen + kConvTile - 1) / kConvTile),
              static_cast<unsigned>(a.batch));
    if (a.apply_silu)
        hipLaunchKernelGGL((causal_conv1d_w4_kernel<T, VEC, true>), grid, dim3(kConvBlock), 0, a.stream,
                           a.x, a.weight, a.bias, a.doc_start, a.conv_state, a.out, a.seqlen,
                           static_cast<int>(a.dim));
    else
        hipLaunchKernelGGL((causal_conv1d_w4_kernel<T, VEC, false>), grid, dim3(kConvBlock), 0, a.stream,
                           a.x, a.weight, a.bias, a.doc_start, a.conv_state, a.out, a.seqlen,
                           static_cast<int>(a.dim));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvArgs& a) {
    if (a.bf16) {
        return a.vectorized ? launch_conv_vec<bf16_t, 8>(a) : launch_conv_vec<bf16_t, 1>(a);
    }
    return a.vectorized ? launch_conv_vec<float, 4>(a) : launch_conv_vec<float, 1>(a);
}

}  // namespace mamba
