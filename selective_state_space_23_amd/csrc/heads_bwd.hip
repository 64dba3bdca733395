// Backward of the scalar-A heads scan (the Mamba-2 shape), gfx950.
//
// What it computes: the gradients of sum(dout * out) + sum(d_final_state *
// final_state) through the scan of scan.hip / ssd.hip with one scalar A per
// head (Mamba skill page, "Mamba-2: Structured State Space Duality (SSD)"; the
// per-document restart of the axolotl page), for u, delta, A, B, C, D, z,
// delta_bias and the initial state.  As the forward's matrix form, it regroups
// the recurrence per chunk of Q = 16 tokens of one (row b, head h): with
// dt_t = softplus(delta_t + bias), cs_t = A (dt_0 + ... + dt_t) (inside the
// chunk), seg_t = document starts in [0, t], H the N x P state entering the
// chunk and x = u (Q x P),
//   L[t, s]  = exp(cs_t - cs_s) if s <= t and seg_s == seg_t, else 0
//   M[t, s]  = (C_t . B_s) L[t, s] dt_s,   scale_t = exp(cs_t) [seg_t == 0]
//   Y        = M x + diag(scale) C H,       out = (Y + D x) silu(z)
//   W_s      = exp(cs_{Q-1} - cs_s) dt_s [seg_s == seg_{Q-1}],   g = scale_{Q-1}
//   H_out    = g H + (diag(W) B)^T x.
// Its adjoint, with dY = dout silu(z) and dH the gradient at H_out:
//   dx  = M^T dY + diag(W) B dH + D dY          dH_in = g dH + C^T diag(scale) dY
//   dM  = dY x^T,  dS = dM o L o dt_s           dC = dS B + diag(scale) dY H^T
//   dB  = dS^T C + diag(W) x dH^T               dz = dout (Y + D x) silu'(z)
// and the scalar chain through cs: dcs_t = sum_s (dM o M)[t, s] - sum_s (dM o M)[s, t]
// + scale_t (dY_t . (C H)_t) - W_t dW_t + [t = Q-1] (g <dH, H> + sum_s W_s dW_s)
// with dW_s = x_s . (B dH)_s; then ddt_s = sum_t dM[t, s] (C_t . B_s) L[t, s]
// + dW_s exp(cs_{Q-1} - cs_s) [seg] + A sum_{t >= s} dcs_t, dA = sum_t dcs_t
// (dt_0 + ... + dt_t), ddelta = ddt softplus'(delta + bias).  The states are
// recomputed, not stored per token ("Hardware-Aware Parallel Scan": recompute in
// the backward); everything runs in fp32, on v_mfma_f32_16x16x4f32 for the
// products (the sums dA, ddelta_bias over tens of thousands of tokens cancel
// heavily, and bf16 operands would show there).
//
// Launches, on segments of the row (one workgroup of 8 waves per (row, head,
// segment)):
//   1. forward pass: each segment from a zero state, chunk by chunk; stores the
//      state entering every chunk (relative to the segment start) and the decay
//      from the segment start, the segment's end state and total decay, and its
//      reverse aggregate X = sum_k (g_0 ... g_{k-1}) C_k^T diag(scale_k) dY_k (the
//      gradient leaving the segment start when none enters its end);
//   2. carries: states entering each segment from the initial state (forward),
//      gradients at each segment end from d_final_state (backward), and the
//      gradient leaving the row start (d_initial_state);
//   3. main pass: each segment chunk by chunk from its last, dH in LDS;
//   4. fixed-order sums over heads (dB, dC) and over rows and segments (dA, dD,
//      ddelta_bias): repeated calls give bitwise identical results.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQ = 16;              // tokens per chunk: one MFMA tile along the tokens
constexpr int kThreads = 512;       // 8 waves: two per SIMD (one 112 KB workgroup per CU)
constexpr int kWaves = kThreads / 64;
static_assert(kWaves == 8, "the wave roles of the main pass assume 8 waves");
constexpr int64_t kTargetBlocks = 768;

struct HbParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* delta_bias;
    const uint8_t* doc_start;
    const float* init;         // (B, D, N) or null
    const void* dout;
    const float* d_final;      // (B, D, N) or null
    void* du;
    void* ddelta;
    void* dz;
    float* d_init;             // (B, D, N) or null
    float* ck;                 // [bh][nck][N][P]: state entering each chunk, from zero at its segment start
    float* gin;                // [bh][nck]: decay from the segment start to the chunk start
    float* hseg;               // [bh][nseg][N][P]: segment end state from zero, then the state entering it
    float* gseg;               // [bh][nseg]: decay over the segment (0 if a document starts in it)
    float* xseg;               // [bh][nseg][N][P]: reverse aggregate, then the gradient at the segment end
    float* dB_part;            // [B][H][L][N]
    float* dC_part;            // [B][H][L][N]
    float* dA_part;            // [bh][nseg]
    float* dbias_part;         // [bh][nseg]
    float* dD_part;            // [bh][nseg][P]
    int64_t seqlen;
    int64_t seg_len;           // multiple of kQ
    int64_t nck;               // chunks per row
    int dim;
    int nheads;
    int nseg;
    int nbatch;
    int softplus;
    int has_z;
};

// acc += X Y for one 16 x 16 tile, K a multiple of 4: X (16 x K) with element
// (i, k) at X[i xi + k xk], Y (K x 16) with element (k, j) at Y[k yk + j yj].
// v_mfma_f32_16x16x4f32: lane l supplies X[l % 16][k0 + l / 16] and
// Y[k0 + l / 16][l % 16]; the result element (4 (l / 16) + e, l % 16) is acc[e].
// SX: 0 plain, 1 X(i, k) scaled by sx[k], 2 by sx[i].
template <int K, int SX = 0>
__device__ __forceinline__ f32x4_t mm(const float* X, int xi, int xk, const float* Y, int yk, int yj, f32x4_t acc,
                                      const float* sx = nullptr) {
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
    // 8 products per trip: enough loads in flight without hoisting all 2 K / 4
    // operands into registers at once
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4) {
        float a = X[r * xi + (k0 + q) * xk];
        if constexpr (SX == 1) a *= sx[k0 + q];
        if constexpr (SX == 2) a *= sx[r];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Y[(k0 + q) * yk + r * yj], acc, 0, 0, 0);
    }
    return acc;
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return Elem<T>::load(p, i);
}

// Per-token scalars of one chunk (lane t < 16 of the calling wave computes token
// t; the others compute nothing useful).  cs is in base-2 units (log2 e A sum dt).
struct ChunkScalars {
    float dt, cs2, S, scale, wexp, W, pre;
    int seg;
    bool valid;
};

template <typename T>
__device__ ChunkScalars chunk_scalars(const HbParams& p, int b, int h, int64_t t0, float a_l2, float dbias) {
    const int lane = threadIdx.x & 63;
    ChunkScalars s;
    const int64_t t = t0 + (lane & 15);
    s.valid = lane < kQ && t < p.seqlen;
    const int64_t tt = s.valid ? t : 0;
    const float raw = ld<T>(p.delta, (static_cast<int64_t>(b) * p.seqlen + tt) * p.nheads + h);
    s.pre = raw + dbias;
    float dt = p.softplus ? softplus_f(s.pre) : s.pre;
    s.dt = s.valid ? dt : 0.0f;
    const bool start = s.valid && ((t == 0 && p.init == nullptr) ||
                                   (p.doc_start != nullptr && p.doc_start[static_cast<int64_t>(b) * p.seqlen + t] != 0));
    // inclusive sum of dt over the 16 tokens (lanes 0..15 of the wave)
    const float S = row16_prefix_sum(s.dt);
    s.S = S;
    s.cs2 = S * a_l2;
    const uint64_t m = __ballot(start) & 0xffffull;
    s.seg = __popcll(m & ((2ull << (lane & 15)) - 1ull));
    const int seg_end = __popcll(m);
    const float cs_end = lane_value(s.cs2, 15);
    s.scale = s.seg == 0 ? exp2_fast(s.cs2) : 0.0f;
    s.wexp = s.seg == seg_end ? exp2_fast(cs_end - s.cs2) : 0.0f;
    s.W = s.wexp * s.dt;
    return s;
}

// Row padding of the LDS tiles, in floats (the [*][N] and [*][P] rows take
// float4 stores, so their padding stays a multiple of 4).
#ifndef MAMBA_HB_PAD_N
#define MAMBA_HB_PAD_N 4
#endif
#ifndef MAMBA_HB_PAD_P
#define MAMBA_HB_PAD_P 4
#endif
#ifndef MAMBA_HB_PAD_Q
#define MAMBA_HB_PAD_Q 1
#endif

// LDS layout of a workgroup (floats).
template <int NT, int P>
struct HbLds {
    static_assert(MAMBA_HB_PAD_N % 4 == 0 && MAMBA_HB_PAD_P % 4 == 0, "float4 rows");
    static constexpr int LN = NT + MAMBA_HB_PAD_N, LP = P + MAMBA_HB_PAD_P, LQ = kQ + MAMBA_HB_PAD_Q;
    static constexpr int oB = 0;                       // B   [Q][LN]
    static constexpr int oC = oB + kQ * LN;             // C   [Q][LN]
    static constexpr int oX = oC + kQ * LN;             // x   [Q][LP]
    static constexpr int oDY = oX + kQ * LP;            // dY  [Q][LP]
    static constexpr int oH = oDY + kQ * LP;            // H   [NT][LP] state entering the chunk
    static constexpr int odH = oH + NT * LP;            // dH  [NT][LP] gradient at the chunk's end state
    static constexpr int oCH = odH + NT * LP;           // C H  [Q][LP]
    static constexpr int oBdH = oCH + kQ * LP;          // B dH [Q][LP]
    static constexpr int oCB = oBdH + kQ * LP;          // C B^T [Q][LQ]
    static constexpr int odM = oCB + kQ * LQ;           // dY x^T [Q][LQ]
    static constexpr int oM = odM + kQ * LQ;            // M  [Q][LQ]
    static constexpr int odS = oM + kQ * LQ;            // dS [Q][LQ]
    static constexpr int oE = odS + kQ * LQ;            // dM o M [Q][LQ]
    static constexpr int oT1 = oE + kQ * LQ;            // dM o (C B^T) o L [Q][LQ]
    static constexpr int oSc = oT1 + kQ * LQ;           // per-token scalars: 8 x Q
    static constexpr int oRed = oSc + 8 * kQ;           // block reduction [kThreads]
    static constexpr int kFloats = oRed + kThreads;
};

// Stage one chunk's B, C rows (Q x NT) and x, dY = dout silu(z) (Q x P) into
// LDS as fp32; tokens past the segment end read as zeros.  Every thread issues
// all of its 16-byte loads before its first LDS store, so their latencies
// overlap (element loads interleaved with LDS stores go one latency at a time:
// a flat load may alias LDS, so none can move above the previous store).
// `between()` runs after the loads are issued: global stores placed there do
// not hold up the wait for these loads (a wave's loads and stores retire in
// issue order), and have the rest of the chunk's work to drain before the next
// chunk's loads.
template <typename T, int NT, int P, typename Between>
__device__ __forceinline__ void stage_chunk(const HbParams& p, int b, int h, int64_t t0, int64_t t_end, float* sB,
                                            float* sC, float* sX, float* sDY, int tid, Between between) {
    using Lay = HbLds<NT, P>;
    constexpr int LN = Lay::LN, LP = Lay::LP;
    constexpr int VEC = 16 / Elem<T>::kBytes;            // elements per 16-byte load
    constexpr int kBC = kQ * NT / VEC;                   // vectors per B or C chunk
    constexpr int kBCit = (2 * kBC + kThreads - 1) / kThreads;
    constexpr int kXv = kQ * P / VEC;                    // vectors per x or dout chunk
    static_assert(kXv <= kThreads, "one x vector per thread");
    const int64_t L = p.seqlen;
    float bc[kBCit][VEC];
#pragma unroll
    for (int k = 0; k < kBCit; ++k) {
        const int i = tid + kThreads * k;
        if (i < 2 * kBC) {
            const int e = (i % kBC) * VEC, t = e / NT, n = e % NT;
            const int64_t tg = t0 + t < t_end ? t0 + t : t0;
            VecIO<T, VEC>::load(i < kBC ? p.B : p.C, (static_cast<int64_t>(b) * L + tg) * NT + n, bc[k]);
        }
    }
    float xv[VEC], dv[VEC], zv[VEC];
    const bool xl = tid < kXv;
    const int xe = (xl ? tid : 0) * VEC, xt = xe / P, xc = xe % P;
    const int64_t xo = (static_cast<int64_t>(b) * L + (t0 + xt < t_end ? t0 + xt : t0)) * p.dim + h * P + xc;
    if (xl) {
        VecIO<T, VEC>::load(p.u, xo, xv);
        VecIO<T, VEC>::load(p.dout, xo, dv);
        if (p.has_z) VecIO<T, VEC>::load(p.z, xo, zv);
    }
    between();
#pragma unroll
    for (int k = 0; k < kBCit; ++k) {
        const int i = tid + kThreads * k;
        if (i < 2 * kBC) {
            const int e = (i % kBC) * VEC, t = e / NT, n = e % NT;
            const bool v = t0 + t < t_end;
            float* dst = (i < kBC ? sB : sC) + t * LN + n;
#pragma unroll
            for (int j = 0; j < VEC; j += 4)
                *reinterpret_cast<float4*>(dst + j) = v ? make_float4(bc[k][j], bc[k][j + 1], bc[k][j + 2], bc[k][j + 3])
                                                        : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
    if (xl) {
        const bool v = t0 + xt < t_end;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            float dy = dv[j];
            if (p.has_z) dy *= silu_f(zv[j]);
            xv[j] = v ? xv[j] : 0.0f;
            dv[j] = v ? dy : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < VEC; j += 4) {
            *reinterpret_cast<float4*>(sX + xt * LP + xc + j) = make_float4(xv[j], xv[j + 1], xv[j + 2], xv[j + 3]);
            *reinterpret_cast<float4*>(sDY + xt * LP + xc + j) = make_float4(dv[j], dv[j + 1], dv[j + 2], dv[j + 3]);
        }
    }
}

// ---------------------------------------------------------------------------
// 1. forward pass over one segment
// ---------------------------------------------------------------------------
template <typename T, int NT, int P>
__global__ __launch_bounds__(kThreads) void heads_bwd_fwd_kernel(const HbParams p) {
    using Lay = HbLds<NT, P>;
    constexpr int LN = Lay::LN, LP = Lay::LP;
    constexpr int kTN = NT / 16, kTP = P / 16, kT = kTN * kTP;
    constexpr int kSt = (kT + kWaves - 1) / kWaves;
    // Only the staged chunk and the scalars (the main pass's layout up to its
    // state tiles): 25 KB at N = 128, P = 64, so two workgroups fit a CU.
    __shared__ float lds[Lay::oH + 3 * kQ];
    float* sB = lds + Lay::oB;
    float* sC = lds + Lay::oC;
    float* sX = lds + Lay::oX;
    float* sDY = lds + Lay::oDY;
    float* sSc = lds + Lay::oH;       // rows: 0 dt, 1 scale, 2 W
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = blockIdx.x;
    const int h = li % p.nheads, seg = (li / p.nheads) % p.nseg, b = li / (p.nheads * p.nseg);
    const int64_t bh = static_cast<int64_t>(b) * p.nheads + h;
    const int64_t L = p.seqlen;
    const int64_t t_seg0 = seg * p.seg_len;
    const int64_t t_seg1 = t_seg0 + p.seg_len < L ? t_seg0 + p.seg_len : L;
    const float a_l2 = p.A[h] * kLog2e;
    const float dbias = p.delta_bias ? p.delta_bias[h] : 0.0f;
    const int64_t PN = static_cast<int64_t>(NT) * P;

    f32x4_t Hs[kSt], Xs[kSt];
#pragma unroll
    for (int j = 0; j < kSt; ++j) {
        Hs[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        Xs[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float G = 1.0f;
    const int r = lane & 15, q = lane >> 4;
    for (int64_t t0 = t_seg0; t0 < t_seg1; t0 += kQ) {
        const int64_t ci = t0 / kQ;
        // the state entering this chunk (relative to the segment start) and its
        // decay, stored once the chunk's loads are on their way
        auto store_entry = [&]() {
            float* ckp = p.ck + (bh * p.nck + ci) * PN;
#pragma unroll
            for (int j = 0; j < kSt; ++j) {
                const int k = wave + kWaves * j;
                if (k < kT) {
                    const int nb = k / kTP, pb = k % kTP;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ckp[(16 * nb + 4 * q + e) * P + 16 * pb + r] = Hs[j][e];
                }
            }
            if (tid == 0) p.gin[bh * p.nck + ci] = G;
        };
        stage_chunk<T, NT, P>(p, b, h, t0, t_seg1, sB, sC, sX, sDY, tid, store_entry);
        if (wave == 0) {
            const ChunkScalars s = chunk_scalars<T>(p, b, h, t0, a_l2, dbias);
            if (lane < kQ) {
                sSc[0 * kQ + lane] = s.dt;
                sSc[1 * kQ + lane] = s.scale;
                sSc[2 * kQ + lane] = s.W;
            }
        }
        lds_barrier();
        const float g = sSc[1 * kQ + kQ - 1];
        // H <- g H + (diag(W) B)^T x;  X += G C^T diag(scale) dY
#pragma unroll
        for (int j = 0; j < kSt; ++j) {
            const int k = wave + kWaves * j;
            if (k < kT) {
                const int nb = k / kTP, pb = k % kTP;
                Hs[j] *= g;
                Hs[j] = mm<kQ, 1>(sB + 16 * nb, 1, LN, sX + 16 * pb, LP, 1, Hs[j], sSc + 2 * kQ);
                f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
                v = mm<kQ, 1>(sC + 16 * nb, 1, LN, sDY + 16 * pb, LP, 1, v, sSc + 1 * kQ);
                Xs[j] += G * v;
            }
        }
        G *= g;
        lds_barrier();
    }
    float* hs = p.hseg + (bh * p.nseg + seg) * PN;
    float* xs = p.xseg + (bh * p.nseg + seg) * PN;
#pragma unroll
    for (int j = 0; j < kSt; ++j) {
        const int k = wave + kWaves * j;
        if (k < kT) {
            const int nb = k / kTP, pb = k % kTP;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int o = (16 * nb + 4 * q + e) * P + 16 * pb + r;
                hs[o] = Hs[j][e];
                xs[o] = Xs[j][e];
            }
        }
    }
    if (tid == 0) p.gseg[bh * p.nseg + seg] = G;
}

// ---------------------------------------------------------------------------
// 2. carries across segments, per (row, head, state element)
// ---------------------------------------------------------------------------
template <int NT, int P>
__global__ __launch_bounds__(256) void heads_bwd_carry_kernel(const HbParams p) {
    const int64_t PN = static_cast<int64_t>(NT) * P;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nbh = static_cast<int64_t>(p.nbatch) * p.nheads;
    if (i >= nbh * PN) return;
    const int64_t bh = i / PN, e = i % PN;
    const int n = static_cast<int>(e / P), c = static_cast<int>(e % P);
    const int64_t b = bh / p.nheads, h = bh % p.nheads;
    const int64_t sidx = (b * p.dim + h * P + c) * NT + n;     // (B, D, N) layout
    float carry = p.init != nullptr ? p.init[sidx] : 0.0f;
    for (int k = 0; k < p.nseg; ++k) {
        float* hp = p.hseg + (bh * p.nseg + k) * PN + e;
        const float local = *hp;
        *hp = carry;                                            // the state entering segment k
        carry = __builtin_fmaf(p.gseg[bh * p.nseg + k], carry, local);
    }
    float grad = p.d_final != nullptr ? p.d_final[sidx] : 0.0f;
    for (int k = p.nseg - 1; k >= 0; --k) {
        float* xp = p.xseg + (bh * p.nseg + k) * PN + e;
        const float local = *xp;
        *xp = grad;                                             // the gradient at the end of segment k
        grad = __builtin_fmaf(p.gseg[bh * p.nseg + k], grad, local);
    }
    if (p.d_init != nullptr) p.d_init[sidx] = grad;
}

// ---------------------------------------------------------------------------
// 3. main pass over one segment, chunks last to first
// ---------------------------------------------------------------------------
template <typename T, int NT, int P>
__global__ __launch_bounds__(kThreads) void heads_bwd_main_kernel(const HbParams p) {
    using Lay = HbLds<NT, P>;
    constexpr int LN = Lay::LN, LP = Lay::LP, LQ = Lay::LQ;
    constexpr int kTN = NT / 16, kTP = P / 16, kT = kTN * kTP;
    constexpr int kSt = (kT + kWaves - 1) / kWaves;
    __shared__ float lds[Lay::kFloats];
    float* sB = lds + Lay::oB;
    float* sC = lds + Lay::oC;
    float* sX = lds + Lay::oX;
    float* sDY = lds + Lay::oDY;
    float* sH = lds + Lay::oH;
    float* sdH = lds + Lay::odH;
    float* sCH = lds + Lay::oCH;
    float* sBdH = lds + Lay::oBdH;
    float* sCB = lds + Lay::oCB;
    float* sdM = lds + Lay::odM;
    float* sM = lds + Lay::oM;
    float* sdS = lds + Lay::odS;
    float* sE = lds + Lay::oE;
    float* sT1 = lds + Lay::oT1;
    float* sSc = lds + Lay::oSc;      // rows: 0 dt, 1 scale, 2 W, 3 wexp, 4 cs2, 5 S, 6 dscale, 7 dW
    float* sRed = lds + Lay::oRed;
    __shared__ int sSeg[kQ];
    __shared__ float sPre[kQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int li = blockIdx.x;
    const int h = li % p.nheads, seg = (li / p.nheads) % p.nseg, b = li / (p.nheads * p.nseg);
    const int64_t bh = static_cast<int64_t>(b) * p.nheads + h;
    const int64_t L = p.seqlen;
    const int64_t t_seg0 = seg * p.seg_len;
    const int64_t t_seg1 = t_seg0 + p.seg_len < L ? t_seg0 + p.seg_len : L;
    const float A = p.A[h];
    const float a_l2 = A * kLog2e;
    const float dbias = p.delta_bias ? p.delta_bias[h] : 0.0f;
    const int64_t PN = static_cast<int64_t>(NT) * P;
    const float* hin_seg = p.hseg + (bh * p.nseg + seg) * PN;

    // dH at the segment end, and D of this head's channels
    {
        const float4* src = reinterpret_cast<const float4*>(p.xseg + (bh * p.nseg + seg) * PN);
        for (int i = tid; i < NT * P / 4; i += kThreads)
            *reinterpret_cast<float4*>(sdH + (4 * i / P) * LP + (4 * i) % P) = src[i];
    }
    // per-lane sums carried over the chunks
    float dD_acc = 0.0f;                  // channel 16 wave + r of Y tiles (waves < kTP)
    float dA_acc = 0.0f, db_acc = 0.0f;   // wave 0, lanes < 16
    // Waves 0 .. kTP-1 own the Y tiles of channel tile `wave`, waves kTP .. 2 kTP-1
    // the dx tiles of channel tile wave - kTP: both need D of that tile.
    const int ptile = wave % kTP;
    const float Dp = (wave < 2 * kTP && p.D != nullptr) ? p.D[h * P + 16 * ptile + r] : 0.0f;

    const int64_t nck_seg = (t_seg1 - t_seg0 + kQ - 1) / kQ;
    // The state entering each chunk is gin * (state entering the segment) + ck;
    // the segment's part stays in registers for all its chunks.
    constexpr int kH4 = NT * P / 4;                          // float4 of a state
    constexpr int kHv = (kH4 + kThreads - 1) / kThreads;    // per thread
    float4 h4[kHv];
    {
        const float4* hsp = reinterpret_cast<const float4*>(hin_seg);
#pragma unroll
        for (int k = 0; k < kHv; ++k) h4[k] = hsp[tid + kThreads * k < kH4 ? tid + kThreads * k : 0];
    }
    for (int64_t cl = nck_seg - 1; cl >= 0; --cl) {
        const int64_t t0 = t_seg0 + cl * kQ;
        const int64_t ci = t0 / kQ;
        // ---- stage: the state entering the chunk (its loads first), B, C, x, dY, scalars
        {
            const float4* ckp = reinterpret_cast<const float4*>(p.ck + (bh * p.nck + ci) * PN);
            float4 c4[kHv];
#pragma unroll
            for (int k = 0; k < kHv; ++k) c4[k] = ckp[tid + kThreads * k < kH4 ? tid + kThreads * k : 0];
            stage_chunk<T, NT, P>(p, b, h, t0, t_seg1, sB, sC, sX, sDY, tid, [] {});
            const float gi = p.gin[bh * p.nck + ci];
#pragma unroll
            for (int k = 0; k < kHv; ++k) {
                if (tid + kThreads * k >= kH4) break;
                const int i = 4 * (tid + kThreads * k);
                *reinterpret_cast<float4*>(sH + (i / P) * LP + i % P) =
                    make_float4(__builtin_fmaf(gi, h4[k].x, c4[k].x), __builtin_fmaf(gi, h4[k].y, c4[k].y),
                                __builtin_fmaf(gi, h4[k].z, c4[k].z), __builtin_fmaf(gi, h4[k].w, c4[k].w));
            }
        }
        if (wave == 0) {
            const ChunkScalars s = chunk_scalars<T>(p, b, h, t0, a_l2, dbias);
            if (lane < kQ) {
                sSc[0 * kQ + lane] = s.dt;
                sSc[1 * kQ + lane] = s.scale;
                sSc[2 * kQ + lane] = s.W;
                sSc[3 * kQ + lane] = s.wexp;
                sSc[4 * kQ + lane] = s.cs2;
                sSc[5 * kQ + lane] = s.S;
                sSeg[lane] = s.seg;
                sPre[lane] = s.pre;
            }
        }
        lds_barrier();

        // ---- products over the states and channels: C H on waves 0 .. 3, B dH on
        //      waves 4 .. 7 (channel tiles kTP <= 4), C B^T and dY x^T on the two
        //      waves with the least of the rest
        if (wave == 3) {
            f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
            a = mm<NT>(sC, LN, 1, sB, 1, LN, a);                       // C B^T
#pragma unroll
            for (int e = 0; e < 4; ++e) sCB[(4 * q + e) * LQ + r] = a[e];
        } else if (wave == 7) {
            f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
            a = mm<P>(sDY, LP, 1, sX, 1, LP, a);                        // dY x^T
#pragma unroll
            for (int e = 0; e < 4; ++e) sdM[(4 * q + e) * LQ + r] = a[e];
        }
        if (wave < kTP) {
            f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
            a = mm<NT>(sC, LN, 1, sH + 16 * wave, LP, 1, a);            // C H
#pragma unroll
            for (int e = 0; e < 4; ++e) sCH[(4 * q + e) * LP + 16 * wave + r] = a[e];
        } else if (wave >= 4 && wave < 4 + kTP) {
            const int pt = wave - 4;
            f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
            c = mm<NT>(sB, LN, 1, sdH + 16 * pt, LP, 1, c);             // B dH
#pragma unroll
            for (int e = 0; e < 4; ++e) sBdH[(4 * q + e) * LP + 16 * pt + r] = c[e];
        }
        lds_barrier();

        // ---- the Q x Q terms (one element per thread), and the row sums of dY o (C H) and x o (B dH)
        if (tid < kQ * kQ) {
            const int t = tid >> 4, s = tid & 15;
            const bool in = s <= t && sSeg[s] == sSeg[t];
            const float lm = in ? exp2_fast(sSc[4 * kQ + t] - sSc[4 * kQ + s]) : 0.0f;
            const float cb = sCB[t * LQ + s], dm = sdM[t * LQ + s], dts = sSc[0 * kQ + s];
            const float m = cb * lm * dts;
            sM[t * LQ + s] = m;
            sdS[t * LQ + s] = dm * lm * dts;
            sE[t * LQ + s] = dm * m;
            sT1[t * LQ + s] = dm * cb * lm;
        }
        if (wave == 2 || wave == 3) {
            // wave 2: dscale_t = dY_t . (C H)_t; wave 3: dW_s = x_s . (B dH)_s
            const float* U = wave == 2 ? sDY : sX;
            const float* V = wave == 2 ? sCH : sBdH;
            float acc = 0.0f;
            for (int c = q; c < P; c += 4) acc = __builtin_fmaf(U[r * LP + c], V[r * LP + c], acc);
            acc += __shfl_xor(acc, 16, 64);
            acc += __shfl_xor(acc, 32, 64);
            if (q == 0) sSc[(wave == 2 ? 6 : 7) * kQ + r] = acc;
        }
        // <dH, H> for the decay g of the chunk, reduced over the workgroup
        {
            float acc = 0.0f;
            for (int i = tid; i < NT * P; i += kThreads) {
                const int o = (i / P) * LP + i % P;
                acc = __builtin_fmaf(sdH[o], sH[o], acc);
            }
            sRed[tid] = acc;
        }
        lds_barrier();

        // ---- outputs over the tokens: Y tiles (waves 0 .. kTP-1: dz, dD) and dx
        //      tiles (waves kTP .. 2 kTP-1: du) of channel tile `ptile`; dC and dB
        //      tiles (state tiles)
        if (wave < kTP) {
            const int pc = 16 * ptile + r;
            f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
            y = mm<kQ>(sM, LQ, 1, sX + 16 * ptile, LP, 1, y);            // M x
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * q + e;
                const int64_t tg = t0 + t;
                const float xv = sX[t * LP + pc], dyv = sDY[t * LP + pc];
                dD_acc = __builtin_fmaf(dyv, xv, dD_acc);
                if (p.has_z && tg < t_seg1) {
                    const int64_t o = (static_cast<int64_t>(b) * L + tg) * p.dim + h * P + pc;
                    const float yv = __builtin_fmaf(Dp, xv, __builtin_fmaf(sSc[1 * kQ + t], sCH[t * LP + pc], y[e]));
                    const float zv = ld<T>(p.z, o);
                    const float sg = rcp_fast(1.0f + exp2_fast(-zv * kLog2e));
                    const float dsilu = sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f);
                    Elem<T>::store(p.dz, o, ld<T>(p.dout, o) * yv * dsilu);
                }
            }
        } else if (wave < 2 * kTP) {
            const int pc = 16 * ptile + r;
            f32x4_t dx = {0.0f, 0.0f, 0.0f, 0.0f};
            dx = mm<kQ>(sM, 1, LQ, sDY + 16 * ptile, LP, 1, dx);         // M^T dY
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * q + e;
                const int64_t tg = t0 + t;
                if (tg < t_seg1) {
                    const int64_t o = (static_cast<int64_t>(b) * L + tg) * p.dim + h * P + pc;
                    const float dyv = sDY[t * LP + pc];
                    const float du = __builtin_fmaf(Dp, dyv, __builtin_fmaf(sSc[2 * kQ + t], sBdH[t * LP + pc], dx[e]));
                    Elem<T>::store(p.du, o, du);
                }
            }
        }
        for (int nb = wave; nb < kTN; nb += kWaves) {
            f32x4_t dc = {0.0f, 0.0f, 0.0f, 0.0f};
            dc = mm<kQ>(sdS, LQ, 1, sB + 16 * nb, LN, 1, dc);                  // dS B
            dc = mm<P, 2>(sDY, LP, 1, sH + 16 * nb * LP, 1, LP, dc, sSc + 1 * kQ);   // diag(scale) dY H^T
            f32x4_t db = {0.0f, 0.0f, 0.0f, 0.0f};
            db = mm<kQ>(sdS, 1, LQ, sC + 16 * nb, LN, 1, db);                 // dS^T C
            db = mm<P, 2>(sX, LP, 1, sdH + 16 * nb * LP, 1, LP, db, sSc + 2 * kQ);   // diag(W) x dH^T
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * q + e;
                const int64_t tg = t0 + t;
                if (tg < t_seg1) {
                    const int64_t o = ((static_cast<int64_t>(b) * p.nheads + h) * L + tg) * NT + 16 * nb + r;
                    p.dC_part[o] = dc[e];
                    p.dB_part[o] = db[e];
                }
            }
        }
        // ---- the scalar chain (wave 0, lane = token)
        float ddelta = 0.0f;
        if (wave == 0) {
            float dg = 0.0f;
            for (int i = 0; i < kThreads; i += 64) dg += sRed[i + lane];
            for (int off = 32; off > 0; off >>= 1) dg += __shfl_xor(dg, off, 64);
            const int t = lane & 15;
            float rowE = 0.0f, colE = 0.0f, t1 = 0.0f, sumWdW = 0.0f;
            for (int k = 0; k < kQ; ++k) {
                rowE += sE[t * LQ + k];
                colE += sE[k * LQ + t];
                t1 += sT1[k * LQ + t];
                sumWdW = __builtin_fmaf(sSc[2 * kQ + k], sSc[7 * kQ + k], sumWdW);
            }
            const float scale = sSc[1 * kQ + t], W = sSc[2 * kQ + t], dW = sSc[7 * kQ + t];
            const float g = sSc[1 * kQ + kQ - 1];
            float dcs = rowE - colE + sSc[6 * kQ + t] * scale - W * dW;
            if (t == kQ - 1) dcs += dg * g + sumWdW;
            // A sum_{t' >= t} dcs_t'
            const float rev = row16_suffix_sum(dcs);
            float ddt = t1 + dW * sSc[3 * kQ + t] + A * rev;
            const bool valid = lane < kQ && t0 + t < t_seg1;
            if (p.softplus) ddt *= rcp_fast(1.0f + exp2_fast(-sPre[t] * kLog2e));
            ddelta = valid ? ddt : 0.0f;
            if (valid) Elem<T>::store(p.ddelta, (static_cast<int64_t>(b) * L + t0 + t) * p.nheads + h, ddt);
            float da = lane < kQ ? dcs * sSc[5 * kQ + t] : 0.0f;
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) {
                da += __shfl_xor(da, off, 64);
                ddelta += __shfl_xor(ddelta, off, 64);
            }
            dA_acc += da;
            db_acc += ddelta;
        }
        lds_barrier();

        // ---- the gradient leaving the chunk start: dH <- g dH + C^T diag(scale) dY
        {
            const float g = sSc[1 * kQ + kQ - 1];
#pragma unroll
            for (int j = 0; j < kSt; ++j) {
                const int k = wave + kWaves * j;
                if (k < kT) {
                    const int nb = k / kTP, pb = k % kTP;
                    f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
                    a = mm<kQ, 1>(sC + 16 * nb, 1, LN, sDY + 16 * pb, LP, 1, a, sSc + 1 * kQ);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float* d = sdH + (16 * nb + 4 * q + e) * LP + 16 * pb + r;
                        *d = __builtin_fmaf(g, *d, a[e]);
                    }
                }
            }
        }
        lds_barrier();
    }

    // partial sums of this (row, head, segment)
    if (wave < kTP) {
        float v = dD_acc;
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (q == 0) p.dD_part[(bh * p.nseg + seg) * P + 16 * wave + r] = v;
    }
    if (tid == 0) {
        p.dA_part[bh * p.nseg + seg] = dA_acc;
        p.dbias_part[bh * p.nseg + seg] = db_acc;
    }
}

// ---------------------------------------------------------------------------
// 4. sums in a fixed order
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void heads_bwd_reduce_bc_kernel(const float* __restrict__ dB_part,
                                                                  const float* __restrict__ dC_part, void* dB, void* dC,
                                                                  int64_t nb, int64_t L, int nheads, int64_t N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;     // over (b, t, n)
    if (i >= nb * L * N) return;
    const int64_t b = i / (L * N), tn = i % (L * N);
    float sb = 0.0f, sc = 0.0f;
    for (int h = 0; h < nheads; ++h) {
        const int64_t o = (b * nheads + h) * L * N + tn;
        sb += dB_part[o];
        sc += dC_part[o];
    }
    Elem<T>::store(dB, i, sb);
    Elem<T>::store(dC, i, sc);
}

__global__ __launch_bounds__(256) void heads_bwd_reduce_w_kernel(const HbParams p, float* dA, float* dD,
                                                                 float* ddelta_bias, int P) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < p.nheads) {
        float a = 0.0f, c = 0.0f;
        for (int b = 0; b < p.nbatch; ++b)
            for (int s = 0; s < p.nseg; ++s) {
                const int64_t k = (static_cast<int64_t>(b) * p.nheads + i) * p.nseg + s;
                a += p.dA_part[k];
                c += p.dbias_part[k];
            }
        dA[i] = a;
        if (ddelta_bias != nullptr) ddelta_bias[i] = c;
    }
    if (dD != nullptr && i < p.dim) {
        const int h = i / P, c = i % P;
        float d = 0.0f;
        for (int b = 0; b < p.nbatch; ++b)
            for (int s = 0; s < p.nseg; ++s)
                d += p.dD_part[((static_cast<int64_t>(b) * p.nheads + h) * p.nseg + s) * P + c];
        dD[i] = d;
    }
}

struct HbPlan {
    int nseg;
    int64_t seg_len;
    int64_t nck;
};

HbPlan plan_heads_bwd(int64_t batch, int64_t seqlen, int nheads) {
    HbPlan s{1, kQ, 0};
    if (seqlen <= 0) return s;
    s.nck = (seqlen + kQ - 1) / kQ;
    const int64_t bh = batch * nheads;
    int64_t want = bh > 0 ? (kTargetBlocks + bh - 1) / bh : 1;
    if (want > s.nck) want = s.nck;
    if (want < 1) want = 1;
    s.seg_len = (s.nck + want - 1) / want * kQ;
    s.nseg = static_cast<int>((seqlen + s.seg_len - 1) / s.seg_len);
    return s;
}

struct HbLayout {
    size_t ck, gin, hseg, gseg, xseg, dB, dC, dA, dbias, dD, total;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

HbLayout hb_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t N, int nheads) {
    const HbPlan pl = plan_heads_bwd(batch, seqlen, nheads);
    const int64_t bh = batch * nheads, P = nheads > 0 ? dim / nheads : 0;
    const size_t pn = static_cast<size_t>(N * P) * 4;
    HbLayout w{};
    size_t off = 0;
    w.ck = off; off += al256(static_cast<size_t>(bh * pl.nck) * pn);
    w.gin = off; off += al256(static_cast<size_t>(bh * pl.nck) * 4);
    w.hseg = off; off += al256(static_cast<size_t>(bh * pl.nseg) * pn);
    w.gseg = off; off += al256(static_cast<size_t>(bh * pl.nseg) * 4);
    w.xseg = off; off += al256(static_cast<size_t>(bh * pl.nseg) * pn);
    w.dB = off; off += al256(static_cast<size_t>(bh * seqlen * N) * 4);
    w.dC = off; off += al256(static_cast<size_t>(bh * seqlen * N) * 4);
    w.dA = off; off += al256(static_cast<size_t>(bh * pl.nseg) * 4);
    w.dbias = off; off += al256(static_cast<size_t>(bh * pl.nseg) * 4);
    w.dD = off; off += al256(static_cast<size_t>(bh * pl.nseg * P) * 4);
    w.total = off;
    return w;
}

template <typename T, int NT, int P>
hipError_t launch_hb_typed(const ScanBwdArgs& a) {
    const HbPlan pl = plan_heads_bwd(a.batch, a.seqlen, a.nheads);
    const HbLayout w = hb_layout(a.batch, a.seqlen, a.dim, NT, a.nheads);
    char* ws = static_cast<char*>(a.ws);
    HbParams p;
    p.u = a.u; p.delta = a.delta; p.A = a.A; p.B = a.B; p.C = a.C; p.D = a.D; p.z = a.z;
    p.delta_bias = a.delta_bias; p.doc_start = a.doc_start; p.init = a.initial_state; p.dout = a.dout;
    p.d_final = a.d_final_state; p.du = a.du; p.ddelta = a.ddelta; p.dz = a.dz; p.d_init = a.d_initial_state;
    p.ck = reinterpret_cast<float*>(ws + w.ck);
    p.gin = reinterpret_cast<float*>(ws + w.gin);
    p.hseg = reinterpret_cast<float*>(ws + w.hseg);
    p.gseg = reinterpret_cast<float*>(ws + w.gseg);
    p.xseg = reinterpret_cast<float*>(ws + w.xseg);
    p.dB_part = reinterpret_cast<float*>(ws + w.dB);
    p.dC_part = reinterpret_cast<float*>(ws + w.dC);
    p.dA_part = reinterpret_cast<float*>(ws + w.dA);
    p.dbias_part = reinterpret_cast<float*>(ws + w.dbias);
    p.dD_part = reinterpret_cast<float*>(ws + w.dD);
    p.seqlen = a.seqlen;
    p.seg_len = pl.seg_len;
    p.nck = pl.nck;
    p.dim = static_cast<int>(a.dim);
    p.nheads = a.nheads;
    p.nseg = pl.nseg;
    p.nbatch = static_cast<int>(a.batch);
    p.softplus = a.softplus ? 1 : 0;
    p.has_z = a.z != nullptr ? 1 : 0;
    const unsigned blocks = static_cast<unsigned>(a.batch * a.nheads * pl.nseg);
    hipLaunchKernelGGL((heads_bwd_fwd_kernel<T, NT, P>), dim3(blocks), dim3(kThreads), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t cnt = a.batch * a.nheads * NT * P;
    hipLaunchKernelGGL((heads_bwd_carry_kernel<NT, P>), dim3(static_cast<unsigned>((cnt + 255) / 256)), dim3(256), 0,
                       a.stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((heads_bwd_main_kernel<T, NT, P>), dim3(blocks), dim3(kThreads), 0, a.stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nbc = a.batch * a.seqlen * NT;
    hipLaunchKernelGGL((heads_bwd_reduce_bc_kernel<T>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0,
                       a.stream, p.dB_part, p.dC_part, a.dB, a.dC, a.batch, a.seqlen, a.nheads, int64_t(NT));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nw = static_cast<int>(a.dim > a.nheads ? a.dim : a.nheads);
    hipLaunchKernelGGL(heads_bwd_reduce_w_kernel, dim3(static_cast<unsigned>((nw + 255) / 256)), dim3(256), 0,
                       a.stream, p, a.dA, a.dD, a.ddelta_bias, P);
    return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_hb_p(const ScanBwdArgs& a) {
    switch (a.dstate) {
        case 16: return launch_hb_typed<T, 16, P>(a);
        case 32: return launch_hb_typed<T, 32, P>(a);
        case 64: return launch_hb_typed<T, 64, P>(a);
        case 128: return launch_hb_typed<T, 128, P>(a);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_hb_dtype(const ScanBwdArgs& a) {
    switch (a.dim / a.nheads) {
        case 32: return launch_hb_p<T, 32>(a);
        case 64: return launch_hb_p<T, 64>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t heads_bwd_kernel_dstate(int64_t dim, int64_t dstate, int nheads) {
    if (nheads <= 0 || dim % nheads != 0 || dstate < 1 || dstate > 128) return 0;
    const int64_t P = dim / nheads;
    if (P != 32 && P != 64) return 0;
    for (int64_t nt = 16; nt <= 128; nt *= 2)
        if (dstate <= nt) return nt;
    return 0;
}

size_t heads_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads) {
    return hb_layout(batch, seqlen, dim, dstate, nheads).total;
}

hipError_t launch_heads_bwd(const ScanBwdArgs& a) {
    return a.bf16 ? launch_hb_dtype<bf16_t>(a) : launch_hb_dtype<float>(a);
}

}  // namespace mamba
