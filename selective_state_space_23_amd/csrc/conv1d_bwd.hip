// Backward pass of the depthwise causal conv1d (width 4) + SiLU, gfx950.
//
// What it computes: the gradients of sum(du * u) through the forward of
// conv1d.hip ("Mamba: Selective State Spaces (S6)" section of the Mamba skill
// page; axolotl page: the conv state restarts at every document start).  With
// acc_t = bias + sum_j w[3-j] x_{t-j} over the taps inside token t's document
// and dacc_t = du_t silu'(acc_t) (du_t without SiLU):
//     dx_s      = sum_{j=0..3} dacc_{s+j} w[3-j]   over the j with s inside (s+j)'s document
//     dw[3-j]   = sum_t dacc_t x_{t-j}             over the same taps
//     dbias     = sum_t dacc_t
//
// Mapping: as the forward, each thread owns VEC consecutive channels and a
// tile of 48 tokens.  It walks the tile and the 3 tokens after it once,
// recomputing acc from a 3-token history (cleared at document starts, primed
// from the 3 tokens before the tile) and keeping the not yet complete dx of the
// last 4 tokens in a shift register: token t adds dacc_t w[3-j] to dx_{t-j} for
// the taps that stay inside its document, and dx_{t-3} is then final.  dw and
// dbias are summed over the tile's own tokens into per-tile partials, which a
// second kernel adds in a fixed order.
//
// A row that continues a given history (conv_state: the inputs of tokens -3..-1)
// treats those three as tokens of token 0's document (unless token 0 starts
// one): they feed acc of tokens 0..2, and their own dx (the gradient of the
// history, d_conv_state) comes out of the shift register of the first tile as
// tokens 0..2 complete it.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

// 2 channels = 4 bytes (bf16) or 8 bytes (fp32).
template <> struct VecIO<bf16_t, 2> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[2]) {
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off);
        v[0] = __uint_as_float(raw << 16);
        v[1] = __uint_as_float(raw & 0xffff0000u);
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[2]) {
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + off) =
            pack_bf16x2(v[0], v[1]);
    }
};
template <> struct VecIO<float, 2> {
    __device__ __forceinline__ static void load(const void* base, int64_t off, float (&v)[2]) {
        const float2 raw = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + off);
        v[0] = raw.x;
        v[1] = raw.y;
    }
    __device__ __forceinline__ static void store(void* base, int64_t off, const float (&v)[2]) {
        *reinterpret_cast<float2*>(static_cast<float*>(base) + off) = make_float2(v[0], v[1]);
    }
};

namespace {

constexpr int kTile = 48;          // tokens per thread; kTile + 6 <= 64 for one ballot
constexpr int kBlock = 256;

template <typename T, int VEC, bool SILU>
__global__ __launch_bounds__(kBlock) void conv1d_bwd_kernel(
    const void* __restrict__ x, const float* __restrict__ weight, const float* __restrict__ bias,
    const uint8_t* __restrict__ doc_start, const void* __restrict__ conv_state, const void* __restrict__ du,
    void* __restrict__ dx, float* __restrict__ d_conv_state, float* __restrict__ part, int64_t seqlen, int dim) {
    const int ngroups = (dim + VEC - 1) / VEC;
    const int grp = blockIdx.x * kBlock + threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTile;
    const int64_t b = blockIdx.z;
    const int64_t row = b * seqlen;

    // Document starts of tokens t0-3 .. t0+kTile+2: bit i <-> token t0 - 3 + i.
    const int lane = threadIdx.x & 63;
    const int64_t tl = t0 - 3 + lane;
    bool is_start = false;
    if (lane < kTile + 6 && tl >= 0 && tl < seqlen)
        is_start = (tl == 0 && conv_state == nullptr) || (doc_start != nullptr && doc_start[row + tl] != 0);
    const uint64_t starts = __ballot(is_start);
    if (grp >= ngroups) return;

    const int d0 = grp * VEC;
    float w0[VEC], w1[VEC], w2[VEC], w3[VEC], bs[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        const float* wr = weight + 4 * (d0 + i);
        w0[i] = wr[0]; w1[i] = wr[1]; w2[i] = wr[2]; w3[i] = wr[3];
        bs[i] = bias ? bias[d0 + i] : 0.0f;
    }

    // History x_{t-1}, x_{t-2}, x_{t-3} restricted to token t's document.
    float h1[VEC], h2[VEC], h3[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
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

    // p0..p3: the running dx of tokens t, t-1, t-2, t-3.
    float p1[VEC], p2[VEC], p3[VEC];
    float gw0[VEC], gw1[VEC], gw2[VEC], gw3[VEC], gb[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        p1[i] = p2[i] = p3[i] = 0.0f;
        gw0[i] = gw1[i] = gw2[i] = gw3[i] = gb[i] = 0.0f;
    }
    // Tokens since the latest document start before t0, capped at 3 (token 0 of
    // a row without history is a start, and the history of one that has it
    // belongs to token 0's document: tiles at the row start need no special case).
    int since = 3;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if ((starts >> k) & 1ull) since = 3 - k;
    const int64_t own_end = (t0 + kTile < seqlen) ? t0 + kTile : seqlen;
    // x and du of the next token are fetched while the current one computes.
    auto fetch = [&](int64_t t, float (&xv)[VEC], float (&gv)[VEC]) {
        if (t < seqlen) {
            VecIO<T, VEC>::load(x, (row + t) * dim + d0, xv);
            VecIO<T, VEC>::load(du, (row + t) * dim + d0, gv);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) xv[i] = gv[i] = 0.0f;
        }
    };
    float xn[VEC], gn[VEC];
    fetch(t0, xn, gn);
    for (int64_t t = t0; t < own_end + 3; ++t) {
        const bool in_row = t < seqlen;
        float xv[VEC], gv[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            xv[i] = xn[i];
            gv[i] = gn[i];
        }
        fetch(t + 1, xn, gn);
        if (in_row && ((starts >> (t - t0 + 3)) & 1ull)) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) h1[i] = h2[i] = h3[i] = 0.0f;
            since = 0;
        }
        const bool own = t < own_end;
        const float m1 = since >= 1 ? 1.0f : 0.0f;
        const float m2 = since >= 2 ? 1.0f : 0.0f;
        const float m3 = since >= 3 ? 1.0f : 0.0f;
        float out[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            float acc = __builtin_fmaf(w3[i], xv[i], bs[i]);
            acc = __builtin_fmaf(w2[i], h1[i], acc);
            acc = __builtin_fmaf(w1[i], h2[i], acc);
            acc = __builtin_fmaf(w0[i], h3[i], acc);
            float g = gv[i];
            if constexpr (SILU) {
                const float sg = rcp_fast(1.0f + exp2_fast(-acc * kLog2e));
                g *= sg * __builtin_fmaf(acc, 1.0f - sg, 1.0f);
            }
            if (own) {
                gb[i] += g;
                gw3[i] = __builtin_fmaf(g, xv[i], gw3[i]);
                gw2[i] = __builtin_fmaf(g, h1[i], gw2[i]);
                gw1[i] = __builtin_fmaf(g, h2[i], gw1[i]);
                gw0[i] = __builtin_fmaf(g, h3[i], gw0[i]);
            }
            // dx_{t-3} is complete after token t's tap; shift the others along.
            out[i] = __builtin_fmaf(g * m3, w0[i], p3[i]);
            p3[i] = __builtin_fmaf(g * m2, w1[i], p2[i]);
            p2[i] = __builtin_fmaf(g * m1, w2[i], p1[i]);
            p1[i] = g * w3[i];
            h3[i] = h2[i];
            h2[i] = h1[i];
            h1[i] = xv[i];
        }
        since = since < 3 ? since + 1 : 3;
        const int64_t s = t - 3;
        if (s >= t0 && s < own_end) {
            VecIO<T, VEC>::store(dx, (row + s) * dim + d0, out);
        } else if (s < 0 && d_conv_state != nullptr) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) d_conv_state[(b * dim + d0 + i) * 3 + (3 + s)] = out[i];
        }
    }
    // Per-tile partials: [b][tile][5][D] (dw columns 0..3, then dbias).
    const int64_t ntiles = gridDim.y;
    float* pt = part + ((b * ntiles + blockIdx.y) * 5) * dim + d0;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        if (d0 + i >= dim) break;
        pt[i] = gw0[i];
        pt[dim + i] = gw1[i];
        pt[2 * dim + i] = gw2[i];
        pt[3 * dim + i] = gw3[i];
        pt[4 * dim + i] = gb[i];
    }
}

// dweight (D, 4) and dbias (D,): sums of the per-tile partials.  A block of 1024
// threads covers 64 consecutive outputs (coalesced 256-byte rows) with 16
// threads each; thread g adds the parts g, g + 16, ... with two accumulators,
// and the 16 sums are added in a fixed order.
__global__ __launch_bounds__(1024) void conv1d_bwd_reduce_kernel(const float* __restrict__ part, float* dweight,
                                                                 float* dbias, int64_t nparts, int dim) {
    constexpr int kGroups = 16;
    __shared__ float red[kGroups][64];
    const int64_t nout = 5 * static_cast<int64_t>(dim);
    const int o = threadIdx.x & 63;
    const int g = threadIdx.x >> 6;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + o;
    float s0 = 0.0f, s1 = 0.0f;
    if (e < nout) {
        int64_t i = g;
        for (; i + kGroups < nparts; i += 2 * kGroups) {
            s0 += part[i * nout + e];
            s1 += part[(i + kGroups) * nout + e];
        }
        if (i < nparts) s0 += part[i * nout + e];
    }
    red[g][o] = s0 + s1;
    __syncthreads();
    if (g != 0 || e >= nout) return;
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) tot += red[k][o];
    const int k = static_cast<int>(e / dim);
    const int d = static_cast<int>(e % dim);
    if (k < 4) dweight[static_cast<int64_t>(d) * 4 + k] = tot;
    else if (dbias) dbias[d] = tot;
}

template <typename T, int VEC>
hipError_t launch_conv_bwd_vec(const ConvBwdArgs& a) {
    const int ngroups = static_cast<int>((a.dim + VEC - 1) / VEC);
    const int64_t ntiles = (a.seqlen + kTile - 1) / kTile;
    dim3 grid((ngroups + kBlock - 1) / kBlock, static_cast<unsigned>(ntiles), static_cast<unsigned>(a.batch));
    if (a.apply_silu)
        hipLaunchKernelGGL((conv1d_bwd_kernel<T, VEC, true>), grid, dim3(kBlock), 0, a.stream, a.x, a.weight,
                           a.bias, a.doc_start, a.conv_state, a.du, a.dx, a.d_conv_state, a.ws, a.seqlen,
                           static_cast<int>(a.dim));
    else
        hipLaunchKernelGGL((conv1d_bwd_kernel<T, VEC, false>), grid, dim3(kBlock), 0, a.stream, a.x, a.weight,
                           a.bias, a.doc_start, a.conv_state, a.du, a.dx, a.d_conv_state, a.ws, a.seqlen,
                           static_cast<int>(a.dim));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(conv1d_bwd_reduce_kernel, dim3(static_cast<unsigned>((5 * a.dim + 63) / 64)), dim3(1024), 0,
                       a.stream, static_cast<const float*>(a.ws), a.dweight, a.dbias, a.batch * ntiles,
                       static_cast<int>(a.dim));
    return hipGetLastError();
}

}  // namespace

size_t conv_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim) {
    return static_cast<size_t>(batch * ((seqlen + kTile - 1) / kTile) * 5 * dim) * sizeof(float);
}

// Pairs of channels for either dtype: the history, pending-dx and gradient
// registers of 2 channels leave room for 8 waves per SIMD, which hides the
// loads' latency better than 4 channels a thread at 4 waves (measured 187 vs
// 233 us on the packed 32K workload; fetching 2 or 3 tokens ahead did not help).
hipError_t launch_causal_conv1d_bwd(const ConvBwdArgs& a) {
    constexpr int V = 2;
    if (a.bf16) return a.vectorized ? launch_conv_bwd_vec<bf16_t, V>(a) : launch_conv_bwd_vec<bf16_t, 1>(a);
    return a.vectorized ? launch_conv_bwd_vec<float, V>(a) : launch_conv_bwd_vec<float, 1>(a);
}

}  // namespace mamba
