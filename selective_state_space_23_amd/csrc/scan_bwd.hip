// Selective-scan backward pass for per-channel A (D, N), gfx950.
//
// What it computes: the gradients of sum(dout * out) through the forward of
// scan.hip (Mamba skill page: S6 block diagram and code, "Core Concept" for the
// D term; axolotl page: per-document restart), i.e. the adjoint of the
// recurrence run backwards in time.  Per channel d and state n, with
// a_t = exp(dt_t A[n]) (0 at a document start) and h_t the forward state:
//   dy_t   = dout_t silu(z_t),   dz_t = dout_t y_t silu'(z_t)
//   g_t    = C_t dy_t + a_{t+1} g_{t+1}           (adjoint of h_t; zero past the row end)
//   dC_t  += dy_t h_t,  dB_t += g_t dt_t u_t      (sums over channels)
//   du_t   = D dy_t + dt_t sum_n g_t B_t
//   ddt_t  = u_t sum_n g_t B_t + sum_n A g_t a_t h_{t-1}
//   dA    += dt_t g_t a_t h_{t-1},  dD += dy_t u_t
//   ddelta_t = ddt_t sigmoid(delta_t + delta_bias) (softplus) or ddt_t,  ddelta_bias += ddelta_t
// The states are recomputed, never stored per token ("Hardware-Aware Parallel
// Scan": recomputation in the backward pass instead of keeping the (B, L, D, N)
// trajectory).
//
// Parallel structure, on the forward's chunking of L:
//   1. aggregate pass, one forward sweep per chunk from a zero state: stores
//      a checkpoint before every 16-token block (the local state, the step-size
//      sum since the chunk start and whether a document started since), and per
//      chunk the local end state H_c, R_c = prod of a over the chunk (0 if a
//      document starts in it) and X_c = a_{t0} g_{t0} of the chunk's own
//      adjoint.  X_c needs no reverse sweep: unrolled, it is the sum over the
//      chunk's tokens of (a_{t0} ... a_t) C_t dy_t, a running product and a
//      running sum carried forward;
//   2. forward carry: the state entering chunk c + 1 is R_c carry_c + H_c;
//   3. reverse carry: G_c = X_{c+1} + R_{c+1} G_{c+1}, the adjoint flowing into
//      the last token of chunk c from the right (the same associative operator,
//      run from the row end);
//   4. main pass, per chunk: the true state before a block is the checkpoint
//      plus exp(A sum) * (chunk's carry), or the checkpoint alone if a document
//      started since the chunk start.
//      The blocks are walked last to first: from that checkpoint recompute the
//      state before token 8 (keeping the one before token 4 in LDS), and for
//      each 4-token piece (last first) its start state (4 more steps for the
//      last piece) and its four states, then run the adjoint over them;
//   5. fixed-order reduction of the per-block partial sums (dB, dC) and of the
//      per-chunk partial sums (dA, dD, ddelta_bias): results are deterministic.
//
// Mapping: as in the forward, lanes are channels and keep their N states and
// adjoints in VGPRs, B_t and C_t are staged in LDS per 64-token window, so du,
// ddt and dA are per-lane sums.  dB_t and dC_t are sums over channels: each
// wave adds its 2N per-lane values of a token across its lanes with permlane
// swaps and DPP (no LDS), the 4 waves' sums meet in LDS, and each block writes
// one partial per token.  The main pass reads a 16-token block's per-channel
// inputs (u, dout, z, delta) from LDS, where buffer loads that write LDS
// directly put them while the block after it (in time) is finishing, so the
// memory latency is hidden without holding registers; each block's step sizes
// dt are formed there from delta once it has landed, in float32 (not rounded to
// the I/O dtype: the token sums dA, dD and ddelta_bias cancel and would show
// that rounding), with the arithmetic every pass uses.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

constexpr int kBlk = 256;              // 4 waves, 256 consecutive channels
constexpr int kWaves = kBlk / 64;
constexpr int kWin = 64;               // tokens per staged B/C window
constexpr int kCk = 16;                // tokens per block of the main pass
constexpr int kCkShift = 4;            // a checkpoint before every block: log2(kCk)
constexpr int kPiece = 4;              // tokens per innermost recompute piece
#ifndef MAMBA_BWD_WAVES_PER_EU
#define MAMBA_BWD_WAVES_PER_EU 0        // 0: the default, 2 waves per SIMD for the main pass
#endif
#ifndef MAMBA_BWD_TOKEN_BARRIER
#define MAMBA_BWD_TOKEN_BARRIER 1
#endif
#ifndef MAMBA_BWD_G16
#define MAMBA_BWD_G16 2          // lanes per channel at N = 16
#endif
#ifndef MAMBA_BWD_G8
#define MAMBA_BWD_G8 1           // lanes per channel at N = 8
#endif
#ifndef MAMBA_BWD_ST4_LDS
#define MAMBA_BWD_ST4_LDS 1      // the state before token 4 of a block kept in LDS
#endif

struct BwdKParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* delta_bias;
    const uint8_t* doc_start;
    const void* dout;
    float* h_agg_P;          // [nslots][B][D][N]: R_s, then (forward carry) the state entering chunk s + 1
    float* h_agg_H;          // [nslots][B][D][N]: H_s
    float* ckpt_out;         // checkpoints, written by the aggregate pass
    const float* h_carry;    // [nslots][B][D][N]: state entering chunk s + 1
    float* g_carry;          // [nslots][B][D][N]: X_{s+1}, then G_s
    float* p_rev;            // [nslots][B][D][N]: P_{s+1}
    const float* ckpt;       // [B][nk][N + 2][D]: local checkpoints of the aggregate pass
    float* part_bc;          // [B][L][nblk][2N]: per-block sums of dB_t, dC_t
    float* part_w;           // [B][nchunks][N + 2][D]: per-chunk sums of dA, dD, ddelta_bias
    const float* init;       // (B, D, N) state before token 0, or null (token 0 then starts a document)
    const float* d_final;    // (B, D, N) gradient arriving at the final state, or null
    float* x0;               // [B][D][N]: X_0 and R_0 of chunk 0 (for d_initial_state), or null
    float* r0;
    void* du;
    void* ddelta;
    void* dz;
    int64_t seqlen;
    int64_t chunk_len;
    int64_t nchunks;
    int64_t nslots;
    int64_t nk;
    int dim;
    int nbatch;
    int nblk;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    constexpr int kRsrcWord3 = 0x00020000;        // gfx9 data format: 32-bit, raw access
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <typename T>
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    if constexpr (sizeof(T) == 2) {
        const uint16_t v = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, byte_off, 0, 0));
        return bf16_to_f32(v);
    } else {
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, 0)));
    }
}

// Element at byte offset voff + soff (soff wave-uniform).
template <typename T>
__device__ __forceinline__ float buf_load_s(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    if constexpr (sizeof(T) == 2) {
        const uint16_t v = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0));
        return bf16_to_f32(v);
    } else {
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0)));
    }
}

template <typename T>
__device__ __forceinline__ void buf_store_s(__amdgpu_buffer_rsrc_t rs, int voff, int soff, float v) {
    if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rs, voff, soff, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, voff, soff, 0);
}

__device__ __forceinline__ float sigmoid_f(float v) { return rcp_fast(1.0f + exp2_fast(-v * kLog2e)); }

// A copy of v the compiler cannot see through.  The recompute levels evaluate the
// same expressions on the same inputs; without this the compiler merges them back
// into one sweep and keeps every intermediate state live (which is exactly what
// recomputation avoids).
__device__ __forceinline__ float opaque(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Stage rows w0 .. w0 + 63 of B (and C) into LDS as fp32 (token-major, N floats a
// token); tokens past t_end are clamped to the last token and never read back.
template <typename T, int N, int kRows>
__device__ __forceinline__ void stage_rows(float* smem, const T* B_row, const T* C_row, int64_t w0, int64_t t_end,
                                           int tid) {
    constexpr int kWinFloats = kWin * N;
    for (int i = tid; i < kRows * kWinFloats; i += kBlk) {
        const int tensor = i / kWinFloats;
        const int e = i % kWinFloats;
        const int tok = e / N;
        const int n = e % N;
        const int64_t t = (w0 + tok < t_end) ? w0 + tok : t_end - 1;
        const T* src = (tensor == 0 || kRows == 1 ? B_row : C_row) + t * N + n;
        float v;
        if constexpr (sizeof(T) == 2) v = bf16_to_f32(*reinterpret_cast<const uint16_t*>(src));
        else v = *reinterpret_cast<const float*>(src);
        smem[i] = v;
    }
}

// Wave-uniform bit mask of the document starts among tokens w0 .. w0 + 63.
// Token 0 starts one unless a state is carried into the row.
__device__ __forceinline__ uint64_t window_starts(const uint8_t* ds_row, int64_t w0, int64_t t_end, int lane,
                                                  bool carried) {
    const int64_t tl = w0 + lane;
    bool st = false;
    if (tl < t_end) st = (tl == 0 && !carried) || (ds_row != nullptr && ds_row[tl] != 0);
    return __ballot(st);
}

// ---------------------------------------------------------------------------
// dt of a token from its raw delta (the fp32 arithmetic of the forward pass).
template <bool SOFTPLUS>
__device__ __forceinline__ float step_size(float delta, float bias) {
    const float v = delta + bias;
    return SOFTPLUS ? softplus_f(v) : v;
}

// 1. One forward sweep of chunk blockIdx.y of row blockIdx.z from a zero state
// (lanes are channels, N states in VGPRs, B and C of a 64-token window in LDS).
// It yields, with one exponential per element:
//   - before every 16-token block a local checkpoint: the state reached from zero
//     at the chunk start, the step-size sum since then (since the latest
//     document start), and whether a document started;
//   - the forward aggregate: the end state H_c and R_c = prod of a over the chunk
//     (exactly 0 once a document starts);
//   - the reverse aggregate X_c = a_{t0} g_{t0} of the adjoint g run backwards
//     from zero over the chunk.  Unrolled, X_c = sum_t R_t C_t dy_t with
//     R_t = prod_{s = t0 .. t} a_s: a forward running sum over the same decays
//     (three multiply-adds per element, no exponential).
#ifndef MAMBA_BWD_AGG_WAVES_PER_EU
#define MAMBA_BWD_AGG_WAVES_PER_EU 3     // 155 VGPRs at N = 16, no spills
#endif
template <typename T, int N, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(kBlk) __attribute__((amdgpu_waves_per_eu(MAMBA_BWD_AGG_WAVES_PER_EU))) void bwd_aggregate_kernel(
    const BwdKParams p) {
    constexpr int kWinFloats = kWin * N;
    __shared__ float4 sBC4[2 * kWinFloats / 4];
    float* sBC = reinterpret_cast<float*>(sBC4);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int d = blockIdx.x * kBlk + tid;
    const bool active = d < p.dim;
    const int dc = active ? d : p.dim - 1;
    const int64_t c = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t L = p.seqlen;
    const int64_t t_begin = c * p.chunk_len;
    const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;
    constexpr int kEsz = static_cast<int>(sizeof(T));
    const int64_t act_row = L * p.dim;
    const int64_t rb = act_row * kEsz;
    const __amdgpu_buffer_rsrc_t u_rs = make_rsrc(static_cast<const T*>(p.u) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t dl_rs = make_rsrc(static_cast<const T*>(p.delta) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(static_cast<const T*>(p.dout) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t z_rs = make_rsrc(static_cast<const T*>(HAS_Z ? p.z : p.dout) + b * act_row, rb);
    const T* B_row = static_cast<const T*>(p.B) + b * L * N;
    const T* C_row = static_cast<const T*>(p.C) + b * L * N;
    const uint8_t* ds_row = p.doc_start ? p.doc_start + b * L : nullptr;

    float Al2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) Al2[n] = p.A[static_cast<int64_t>(dc) * N + n] * kLog2e;
    const float dbias = p.delta_bias ? p.delta_bias[dc] : 0.0f;
    const int lane_off = dc * kEsz;
    const int row_bytes = p.dim * kEsz;
    float h[N], R[N], X[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        h[n] = 0.0f;
        R[n] = 1.0f;
        X[n] = 0.0f;
    }
    float sum_dt = 0.0f;
    bool any_reset = false;
    float* ck_row = p.ckpt_out + b * p.nk * (N + 2) * p.dim;

    // u, delta, dout, z of tokens g0 .. g0 + 3 (clamped to the chunk's last token).
    auto fetch = [&](int64_t g0, float (&uu)[kPiece], float (&dl)[kPiece], float (&go)[kPiece],
                     float (&zz)[kPiece]) {
#pragma unroll
        for (int k = 0; k < kPiece; ++k) {
            const int64_t t = g0 + k < t_end ? g0 + k : t_end - 1;
            const int so = static_cast<int>(t * row_bytes);
            uu[k] = buf_load_s<T>(u_rs, lane_off, so);
            dl[k] = buf_load_s<T>(dl_rs, lane_off, so);
            go[k] = buf_load_s<T>(do_rs, lane_off, so);
            zz[k] = HAS_Z ? buf_load_s<T>(z_rs, lane_off, so) : 0.0f;
        }
    };
    uint64_t starts = 0;
    auto steps = [&](int64_t g0, int64_t w0, const float (&uu)[kPiece], const float (&dl)[kPiece],
                     const float (&go)[kPiece], const float (&zz)[kPiece]) {
        // Stores take the clamped channel and token: a lane past the last channel
        // (or a token past the chunk end) repeats the value of the lane (token) it
        // was clamped to, so no store needs a branch inside the token loop.
        if (((g0 - t_begin) & (kCk - 1)) == 0 && g0 < t_end) {
            // One resource per checkpoint: wave-uniform base, row offsets in soffset.
            const __amdgpu_buffer_rsrc_t ck_rs =
                make_rsrc(ck_row + (g0 >> kCkShift) * (N + 2) * p.dim, (N + 2) * p.dim * 4);
#pragma unroll
            for (int n = 0; n < N; ++n) buf_store_s<float>(ck_rs, dc * 4, n * p.dim * 4, h[n]);
            buf_store_s<float>(ck_rs, dc * 4, N * p.dim * 4, sum_dt);
            buf_store_s<float>(ck_rs, dc * 4, (N + 1) * p.dim * 4, any_reset ? 1.0f : 0.0f);
        }
#pragma unroll
        for (int k = 0; k < kPiece; ++k) {
            const int64_t t = g0 + k;
            const bool valid = t < t_end;
            const int o = static_cast<int>(t - w0);
            const bool reset = (starts >> o) & 1ull;
            const float r = reset ? -__builtin_inff() : 0.0f;
            float dt = step_size<SOFTPLUS>(dl[k], dbias);
            dt = valid ? dt : 0.0f;
            float dy = go[k];
            if constexpr (HAS_Z) dy *= silu_f(zz[k]);
            dy = valid ? dy : 0.0f;
            any_reset = any_reset || reset;
            sum_dt = reset ? 0.0f : sum_dt;
            const float w = dt * uu[k];
            const float4* Bq = reinterpret_cast<const float4*>(sBC + o * N);
            const float4* Cq = reinterpret_cast<const float4*>(sBC + kWinFloats + o * N);
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const float4 bv = Bq[q];
                const float4 cv = Cq[q];
                const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
                const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = 4 * q + j;
                    const float a = exp2_fast(__builtin_fmaf(dt, Al2[n], r));
                    h[n] = __builtin_fmaf(a, h[n], w * bb[j]);
                    R[n] *= a;
                    X[n] = __builtin_fmaf(R[n], cc[j] * dy, X[n]);
                }
            }
            // Keep each token's R and X updates in that token (the compiler
            // otherwise defers them over the group and spills the decays).
#pragma unroll
            for (int n = 0; n < N; ++n) {
                R[n] = opaque(R[n]);
                X[n] = opaque(X[n]);
            }
            sum_dt += dt;
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    float au[kPiece], ad[kPiece], ao[kPiece], az[kPiece], bu[kPiece], bd[kPiece], bo[kPiece], bz[kPiece];
    fetch(t_begin, au, ad, ao, az);
    for (int64_t w0 = t_begin; w0 < t_end; w0 += kWin) {
        starts = window_starts(ds_row, w0, t_end, lane, p.init != nullptr);
        __syncthreads();
        stage_rows<T, N, 2>(sBC, B_row, C_row, w0, t_end, tid);
        __syncthreads();
        const int64_t wend = (w0 + kWin < t_end) ? w0 + kWin : t_end;
        for (int64_t g0 = w0; g0 < wend; g0 += 2 * kPiece) {
            fetch(g0 + kPiece, bu, bd, bo, bz);
            steps(g0, w0, au, ad, ao, az);
            fetch(g0 + 2 * kPiece, au, ad, ao, az);
            steps(g0 + kPiece, w0, bu, bd, bo, bz);
        }
    }
    if (!active) return;
    const int64_t count = static_cast<int64_t>(p.nbatch) * p.dim * N;
    const int64_t my_slot = (b * p.dim + d) * N;
    if (c < p.nslots) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            p.h_agg_P[c * count + my_slot + n] = R[n];
            p.h_agg_H[c * count + my_slot + n] = h[n];
        }
    }
    if (c > 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            p.g_carry[(c - 1) * count + my_slot + n] = X[n];
            p.p_rev[(c - 1) * count + my_slot + n] = R[n];
        }
    } else if (p.x0 != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            p.x0[my_slot + n] = X[n];
            p.r0[my_slot + n] = R[n];
        }
    }
}

// 2. Forward carry: slot s turns from R_s into the state entering chunk s + 1,
// carry_{s+1} = R_s carry_s + H_s (carry_0: the initial state, or 0).
__global__ __launch_bounds__(256) void bwd_fwd_carry_kernel(float* __restrict__ ws_P, const float* __restrict__ ws_H,
                                                            const float* __restrict__ init, int64_t count,
                                                            int64_t nslots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= count) return;
    float carry = init != nullptr ? init[i] : 0.0f;
    int64_t s = 0;
    for (; s + 4 <= nslots; s += 4) {
        float P[4], H[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            P[k] = ws_P[(s + k) * count + i];
            H[k] = ws_H[(s + k) * count + i];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            carry = __builtin_fmaf(P[k], carry, H[k]);
            ws_P[(s + k) * count + i] = carry;
        }
    }
    for (; s < nslots; ++s) {
        carry = __builtin_fmaf(ws_P[s * count + i], carry, ws_H[s * count + i]);
        ws_P[s * count + i] = carry;
    }
}

// 3. Reverse carry: slot s turns from X_{s+1} into G_s = X_{s+1} + P_{s+1} G_{s+1},
// starting from the gradient arriving at the final state (or 0) as G of the
// last chunk.  With d_init, the adjoint leaving the row to the left follows:
// d_init = X_0 + R_0 G_0 (the same operator once more, over chunk 0).
__global__ __launch_bounds__(256) void bwd_rev_carry_kernel(float* __restrict__ g_carry,
                                                            const float* __restrict__ p_rev,
                                                            const float* __restrict__ d_final,
                                                            const float* __restrict__ x0, const float* __restrict__ r0,
                                                            float* __restrict__ d_init, int64_t count, int64_t nslots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= count) return;
    float G = d_final != nullptr ? d_final[i] : 0.0f;
    int64_t s = nslots - 1;
    for (; s >= 3; s -= 4) {
        float X[4], P[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            X[k] = g_carry[(s - k) * count + i];
            P[k] = p_rev[(s - k) * count + i];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            G = __builtin_fmaf(P[k], G, X[k]);
            g_carry[(s - k) * count + i] = G;
        }
    }
    for (; s >= 0; --s) {
        G = __builtin_fmaf(p_rev[s * count + i], G, g_carry[s * count + i]);
        g_carry[s * count + i] = G;
    }
    if (d_init != nullptr) d_init[i] = __builtin_fmaf(r0[i], G, x0[i]);
}

// ---------------------------------------------------------------------------
// 4. Main pass over chunk blockIdx.y of row blockIdx.z.
//
// G lanes share one channel, each holding NL = N / G of its states (G = 2 at
// N = 16 halves the per-lane arrays, which is what lets the pass run without
// spills);
// their partial sums over states (g.B, the A term, C.h) meet through one DPP
// exchange per sum, and every lane of the group computes the per-token scalars.
template <int G>
__device__ __forceinline__ float sum_group(float v) {
    if constexpr (G >= 2)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    if constexpr (G >= 4)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    return v;
}

// Sums over lanes without LDS: V values per lane (v[i], v[i + V/2] are dB and dC
// terms of one state), added over the lanes that differ in bits 1..5 of the lane
// index, and over bit 0 too unless HALVES (then lanes l and l ^ 1 hold different
// state halves of one channel and stay apart).  Each step pairs lanes that differ
// in one bit: each keeps half of its values and receives the partner's partial
// sums of that half, so the exchanges halve with every step (the permlane swaps
// of bits 5 and 4 deliver both halves at once).  Lane l ends with the total of
// value (l >> 2) & 15 (V = 16) or (l >> 3) & 7 (V = 8) of its half.
// v_permlane32_swap exchanges lanes 32..63 of a with lanes 0..31 of b, so a + b
// afterwards holds value a summed over lane pairs (l, l + 32) in the low half
// and value b in the high half; v_permlane16_swap does the same for odd and even
// 16-lane rows.  Written as asm because the compiler's builtins for them lose
// the second result (both results come back in one register).  Four swaps share
// one asm block: its leading s_nop gives the VALU-write-to-permlane-read
// distance the compiler cannot see through asm (the swaps inside touch
// different registers), the trailing one separates the last swap from a read
// of its results.
#define MAMBA_SWAP4(op, a, b)                                                                            \
    asm("s_nop 1\n\t" op " %0, %4\n\t" op " %1, %5\n\t" op " %2, %6\n\t" op " %3, %7\n\ts_nop 0"   \
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]))
__device__ __forceinline__ void swap_add32x4(float (&a)[4], float (&b)[4], float* out) {
    MAMBA_SWAP4("v_permlane32_swap_b32", a, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = a[j] + b[j];
}
__device__ __forceinline__ void swap_add16x4(float (&a)[4], float (&b)[4], float* out) {
    MAMBA_SWAP4("v_permlane16_swap_b32", a, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = a[j] + b[j];
}
__device__ __forceinline__ float swap_add16(float a, float b) {
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 0" : "+v"(a), "+v"(b));
    return a + b;
}
__device__ __forceinline__ float dpp_f(float v, int ctrl_is_ror8) {
    return __builtin_bit_cast(float, ctrl_is_ror8
        ? __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)     // lane ^ 8 (row_ror:8)
        : __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));    // lane ^ 2 (quad_perm 2,3,0,1)
}
__device__ __forceinline__ float xor4_f(float v, bool hi) {           // the value of lane ^ 4
    const int a = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xF, 0xF, false);   // lane + 4
    const int b = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, false);   // lane - 4
    return __builtin_bit_cast(float, hi ? b : a);
}
// Steps for bits 5 and 4 on one group of values; used per group of 4 states as
// the values are produced (w[i] = the bit-5 sums, filled in 4 at a time).
template <int V, bool HALVES>
__device__ __forceinline__ float lane_sum_finish(const float (&w)[V / 2], int lane) {
    constexpr int V2 = V / 4;
    float x[V2];
    if constexpr (V2 == 4) {
        float lo[4] = {w[0], w[1], w[2], w[3]}, hi[4] = {w[4], w[5], w[6], w[7]};
        swap_add16x4(lo, hi, x);
    } else {
#pragma unroll
        for (int i = 0; i < V2; ++i) x[i] = swap_add16(w[i], w[i + V2]);
    }
    const bool b3 = lane & 8, b2 = lane & 4;
    float z;
    if constexpr (V2 == 4) {
        float y[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float keep = b3 ? x[i + 2] : x[i];
            const float send = b3 ? x[i] : x[i + 2];
            y[i] = keep + dpp_f(send, 1);
        }
        const float keep = b2 ? y[1] : y[0];
        const float send = b2 ? y[0] : y[1];
        z = keep + xor4_f(send, b2);
    } else {
        static_assert(V2 == 2, "8 or 16 values a lane");
        const float keep = b3 ? x[1] : x[0];
        const float send = b3 ? x[0] : x[1];
        const float y = keep + dpp_f(send, 1);
        z = y + xor4_f(y, b2);
    }
    z += dpp_f(z, 0);
    if constexpr (!HALVES)
        z += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, z), 0xB1, 0xF, 0xF, false));
    return z;
}

// Waves per SIMD the main pass is compiled for: 2, which leaves it the
// registers to run without spills (at 3 the spill traffic missed in L2 and cost
// more than the extra wave hid; its inputs arrive through LDS, so it needs
// little occupancy for latency).
constexpr int kBwdWavesPerEu = MAMBA_BWD_WAVES_PER_EU > 0 ? MAMBA_BWD_WAVES_PER_EU : 2;

template <typename T, int N, int G, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(kBlk) __attribute__((amdgpu_waves_per_eu(kBwdWavesPerEu))) void bwd_chunk_kernel(
    const BwdKParams p) {
    constexpr int NL = N / G;              // states per lane
    constexpr int CPB = kBlk / G;          // channels per block
    constexpr int V = 2 * NL;              // dB_t and dC_t terms of one lane
    constexpr int NOUT = 2 * N;            // sums per token: dB_t, then dC_t
    constexpr int kSumShift = V == 16 ? 2 : 3;              // lane l holds value (l >> kSumShift) of the lane sums
    constexpr int kWriter = ((1 << kSumShift) - 1) & (G == 2 ? ~1 : ~0);   // lanes with (l & kWriter) == 0 store it
    constexpr int kWinFloats = kWin * N;
    static_assert(N % G == 0 && NL % 4 == 0 && G <= 2 && (V == 8 || V == 16), "state split");
    __shared__ float4 sBC4[2 * kWinFloats / 4];          // B then C of the window
    __shared__ float sP[2][kWaves * kCk * NOUT];         // per-wave sums of a 16-token block (2 buffers)
    float* sBC = reinterpret_cast<float*>(sBC4);
    // Per-wave staging of one 16-token block's per-channel inputs, token-major:
    // dt (fp32, formed in place from delta once the block has landed), then u,
    // dout, [z], delta (T) of the wave's CPW channels.
    constexpr int CPW = 64 / G;                                          // channels per wave
    constexpr int kTsz = static_cast<int>(sizeof(T));
    constexpr int kNArr = 3 + (HAS_Z ? 1 : 0);
    constexpr int kStgBytes = kCk * CPW * (4 + kNArr * kTsz);
    static_assert(kStgBytes % 16 == 0, "staging rows");
    __shared__ float4 sStg4[kWaves * kStgBytes / 16];
#if MAMBA_BWD_ST4_LDS
    // The state before token 4 of the current block, saved while the state
    // before token 8 is recomputed: piece 1 starts from it instead of
    // re-advancing tokens 0..3 a third time.  [q][thread] float4s.
    static_assert(NL % 4 == 0, "states in float4s");
    __shared__ float4 sH4[(NL / 4) * kBlk];
#endif

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = tid % G;
    const int n0 = sub * NL;                // first state of this lane
    const int d = blockIdx.x * CPB + tid / G;
    const bool active = d < p.dim;
    const int dc = active ? d : p.dim - 1;
    const int64_t c = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t L = p.seqlen;
    const int64_t t_begin = c * p.chunk_len;
    const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;

    constexpr int kEsz = static_cast<int>(sizeof(T));
    const int64_t act_row = L * p.dim;
    const int64_t rb = act_row * kEsz;
    const __amdgpu_buffer_rsrc_t u_rs = make_rsrc(static_cast<const T*>(p.u) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t dl_rs = make_rsrc(static_cast<const T*>(p.delta) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(static_cast<const T*>(p.dout) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t z_rs = make_rsrc(static_cast<const T*>(HAS_Z ? p.z : p.dout) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t du_rs = make_rsrc(static_cast<T*>(p.du) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t dd_rs = make_rsrc(static_cast<T*>(p.ddelta) + b * act_row, rb);
    const __amdgpu_buffer_rsrc_t dz_rs = make_rsrc(static_cast<T*>(HAS_Z ? p.dz : p.du) + b * act_row, rb);
    const T* B_row = static_cast<const T*>(p.B) + b * L * N;
    const T* C_row = static_cast<const T*>(p.C) + b * L * N;
    const uint8_t* ds_row = p.doc_start ? p.doc_start + b * L : nullptr;

    float Al2[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) Al2[i] = p.A[static_cast<int64_t>(dc) * N + n0 + i] * kLog2e;
    const float dbias = p.delta_bias ? p.delta_bias[dc] : 0.0f;
    const float Dd = p.D ? p.D[dc] : 0.0f;
    const int64_t count = static_cast<int64_t>(p.nbatch) * p.dim * N;
    const int64_t my_slot = (b * p.dim + dc) * N + n0;
    // Checkpoint k of this row: (N + 2) rows of dim floats at ck_row + k (N + 2) dim.
    const float* ck_row = p.ckpt + b * p.nk * (N + 2) * p.dim;

    // Element offsets: a lane-constant byte offset plus a wave-uniform one per
    // token (the buffer instruction's scalar offset), so per-token addresses cost
    // no VGPRs.
    const int lane_off = dc * kEsz;
    const int row_bytes = p.dim * kEsz;
    auto tok_soff = [&](int64_t t) -> int {          // clamped to the chunk's last token
        return static_cast<int>((t < t_end ? t : t_end - 1) * row_bytes);
    };

    uint64_t starts = 0;
    // One forward step of the token at window offset o: h <- exp(dt A) h + w B_t.
    auto fstep = [&](float (&h)[NL], float dt, float w, int o) {
        const float r = ((starts >> o) & 1ull) ? -__builtin_inff() : 0.0f;
        const float4* Bq = reinterpret_cast<const float4*>(sBC + o * N + n0);
#pragma unroll
        for (int q = 0; q < NL / 4; ++q) {
            const float4 bv = Bq[q];
            const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * q + j;
                h[i] = __builtin_fmaf(exp2_fast(__builtin_fmaf(dt, Al2[i], r)), h[i], w * bb[j]);
            }
        }
        // Keep the scheduler from hoisting later tokens' LDS reads and
        // exponentials: each token already offers NL independent chains.
        __builtin_amdgcn_sched_barrier(0);
    };
    // Staging: the wave's inputs of the block at s_cur arrive in LDS through
    // buffer loads that write LDS directly (no registers held while in flight),
    // issued one block ahead.  Lane l of such a load writes the dword at
    // lds + 4 l, so a load covers 64 / CPW (dt) or 64 / (CPW T / 4) (T arrays)
    // token rows: a lane-constant byte offset (row within the load, channel)
    // plus a wave-uniform one for the token.  Channels past the last are clamped
    // to it (their lanes are inactive); tokens past the chunk end read the next
    // chunk's values or, past the row end, zeros (the buffer range check), and
    // are masked where they are used.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    char* stg = reinterpret_cast<char*>(sStg4) + wave_s * kStgBytes;
    const int cw0 = blockIdx.x * CPB + wave_s * CPW;                     // first channel of the wave
    const int chw = lane / G;                                            // this lane's channel in the wave
    auto lds_ptr = [](char* q) { return (__attribute__((address_space(3))) void*)(q); };
    auto stage_voff = [&](int esz) {             // lane-constant part of a staging load's offset
        const int lpr = CPW * esz / 4;          // dwords per token row
        const int ce = (lane % lpr) * (4 / esz);
        const int ch = cw0 + ce < p.dim ? cw0 + ce : p.dim - 4 / esz;
        return ((lane / lpr) * p.dim + ch) * esz;
    };
    const int voff_t = stage_voff(kTsz);
    auto stage_arr = [&](__amdgpu_buffer_rsrc_t rs, int esz, int voff, char* dst, int64_t s0) {
        const int tpi = 64 / (CPW * esz / 4);   // token rows per load
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i * tpi >= kCk) break;
            // The token part goes into the lane (VGPR) offset, not the scalar one:
            // the buffer's range check covers only the former, and the last block
            // of a row reaches up to 15 token rows past the row's end.
            const int v = voff + static_cast<int>((s0 + i * tpi) * p.dim * esz);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst + i * tpi * CPW * esz), 4, v, 0, 0, 0);
        }
    };
    auto stage_block = [&](int64_t s0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this wave's reads of the buffer are done
        char* q = stg + kCk * CPW * 4;          // the dt rows are formed from delta
        stage_arr(u_rs, kTsz, voff_t, q, s0);
        q += kCk * CPW * kTsz;
        stage_arr(do_rs, kTsz, voff_t, q, s0);
        q += kCk * CPW * kTsz;
        if constexpr (HAS_Z) {
            stage_arr(z_rs, kTsz, voff_t, q, s0);
            q += kCk * CPW * kTsz;
        }
        stage_arr(dl_rs, kTsz, voff_t, q, s0);
    };
    auto stg_val = [&](int arr, int k) -> float {          // arr 0: dt, 1: u, 2: dout, 3: z, 4: delta
        if (arr == 0) return reinterpret_cast<const float*>(stg)[k * CPW + chw];
        int slot = arr - 1;
        if (!HAS_Z && arr == 4) slot = 2;
        const char* base = stg + kCk * CPW * 4 + slot * kCk * CPW * kTsz;
        if constexpr (kTsz == 2)
            return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[k * CPW + chw]);
        else
            return reinterpret_cast<const float*>(base)[k * CPW + chw];
    };
    int64_t s_cur = 0;                          // first token of the staged block
    // dt and u of token t of the staged block: dt = 0 past the chunk end (an
    // identity step), u = 0 on an inactive lane (its dB terms vanish).  The
    // values pass through opaque() so that each recompute level evaluates its
    // own exponentials.
    const float active_f = active ? 1.0f : 0.0f;
    auto load_dtu = [&](int64_t t, float& dt, float& uu) {
        const int k = static_cast<int>(t - s_cur);
        dt = opaque(stg_val(0, k) * (t < t_end ? 1.0f : 0.0f));
        uu = stg_val(1, k) * active_f;
    };
    // The state entering the chunk (row b of carry slot c - 1, or of the initial
    // state for chunk 0).
    const bool carried_in = c > 0 || p.init != nullptr;
    const __amdgpu_buffer_rsrc_t hin_rs =
        make_rsrc((c > 0 ? p.h_carry + (c - 1) * count : (p.init != nullptr ? p.init : p.h_carry)) + b * p.dim * N,
                  p.dim * N * 4);
    // The next block's checkpoint rows (local state, step-size sum, document
    // flag), fetched into registers with the block's staging.
    float ckv[NL], hinv[NL], ck_cdt = 0.0f, ck_flag = 0.0f;
    auto fetch_ck = [&](int64_t s0) {
        const __amdgpu_buffer_rsrc_t ck_rs =
            make_rsrc(ck_row + (s0 >> kCkShift) * (N + 2) * p.dim, (N + 2) * p.dim * 4);
#pragma unroll
        for (int i = 0; i < NL; ++i) ckv[i] = buf_load_s<float>(ck_rs, (n0 * p.dim + dc) * 4, i * p.dim * 4);
        ck_cdt = buf_load_s<float>(ck_rs, dc * 4, N * p.dim * 4);
        ck_flag = buf_load_s<float>(ck_rs, dc * 4, (N + 1) * p.dim * 4);
#pragma unroll
        for (int i = 0; i < NL; ++i) hinv[i] = buf_load_s<float>(hin_rs, (dc * N + n0) * 4, i * 4);
    };
    // h <- the state after tokens t0 .. t0 + 3 (window offsets o0 ..).
    auto advance4 = [&](float (&h)[NL], int64_t t0, int o0) {
        float dtv[kPiece], uv[kPiece];
#pragma unroll
        for (int k = 0; k < kPiece; ++k) load_dtu(t0 + k, dtv[k], uv[k]);
#pragma unroll
        for (int k = 0; k < kPiece; ++k) fstep(h, dtv[k], dtv[k] * uv[k], o0 + k);
    };

    float gn[NL];         // a_{t+1} g_{t+1}: the adjoint reaching token t from the right
    if (c + 1 < p.nchunks || p.d_final != nullptr) {
        // (the last chunk: the gradient arriving at the final state)
        const float* gc = (c + 1 < p.nchunks ? p.g_carry + c * count : p.d_final) + my_slot;
#pragma unroll
        for (int i = 0; i < NL; ++i) gn[i] = gc[i];
    } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) gn[i] = 0.0f;
    }
    float dA[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) dA[i] = 0.0f;
    float dD_acc = 0.0f, db_acc = 0.0f;
    int buf = 0;

    // Sum the 4 waves' sums of 16-token block s and store the block's partials.
    auto flush16 = [&](const float* sp, int64_t s) {
        const int64_t nvalid = (s + kCk < t_end) ? kCk : t_end - s;
        for (int e = tid; e < kCk * NOUT; e += kBlk) {
            const int tok = e / NOUT;
            const int j = e % NOUT;
            if (tok < nvalid) {
                float sum = sp[tok * NOUT + j];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) sum += sp[(w * kCk + tok) * NOUT + j];
                p.part_bc[((b * L + s + tok) * p.nblk + blockIdx.x) * NOUT + j] = sum;
            }
        }
    };

    // One 4-token piece starting at s4 (window offset o4, block offset k4) from
    // the state st before it: recompute the four states, then run the adjoint
    // over them, last first.
    auto piece = [&](int64_t s4, int o4, int k4, const float (&st)[NL], float* sp) {
        float dtv[kPiece], uv[kPiece], dov[kPiece], zv[kPiece], dlv[kPiece];
#pragma unroll
        for (int k = 0; k < kPiece; ++k) {
            load_dtu(s4 + k, dtv[k], uv[k]);
            const int kk = static_cast<int>(s4 + k - s_cur);
            dov[k] = stg_val(2, kk);
            zv[k] = HAS_Z ? stg_val(3, kk) : 0.0f;
            dlv[k] = SOFTPLUS ? stg_val(4, kk) : 0.0f;
        }
        // The last piece of a block has read its inputs: the staging buffer is
        // free for the block before it.
        if (s4 == s_cur && s_cur > t_begin) {
            stage_block(s_cur - kCk);
            fetch_ck(s_cur - kCk);
        }
        float hs[kPiece][NL];
#pragma unroll
        for (int k = 0; k < kPiece; ++k) {
#pragma unroll
            for (int i = 0; i < NL; ++i) hs[k][i] = k == 0 ? st[i] : hs[k - 1][i];
            fstep(hs[k], dtv[k], dtv[k] * uv[k], o4 + k);
        }
#pragma unroll
        for (int k = kPiece - 1; k >= 0; --k) {
            const int64_t t = s4 + k;
            const bool live = t < t_end && active;
            const int o = o4 + k;
            const float r = ((starts >> o) & 1ull) ? -__builtin_inff() : 0.0f;
            // The same dt as the recompute above, so the compiler keeps that
            // recompute's decays in registers for the adjoint (4 x NL values).
            const float dt = dtv[k];
            const float uu = uv[k];
            const float w = dt * uu;
            float sgz = 0.0f, dy = dov[k];
            if constexpr (HAS_Z) {
                sgz = sigmoid_f(zv[k]);
                dy *= zv[k] * sgz;
            }
            dy = live ? dy : 0.0f;
            const float4* Bq = reinterpret_cast<const float4*>(sBC + o * N + n0);
            const float4* Cq = reinterpret_cast<const float4*>(sBC + kWinFloats + o * N + n0);
            float sB = 0.0f, sq = 0.0f, y = 0.0f;
            float wsum[NL];        // dB_t and dC_t terms of state i, summed over lane bit 5
#pragma unroll
            for (int q = 0; q < NL / 4; ++q) {
                const float4 bv = Bq[q];
                const float4 cv = Cq[q];
                const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
                const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
                float vb[4], vc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * q + j;
                    const float hprev = k == 0 ? st[i] : hs[k > 0 ? k - 1 : 0][i];
                    const float a = exp2_fast(__builtin_fmaf(dt, Al2[i], r));
                    const float g = __builtin_fmaf(cc[j], dy, gn[i]);
                    gn[i] = a * g;
                    const float gq = g * (a * hprev);
                    sq = __builtin_fmaf(Al2[i], gq, sq);
                    dA[i] = __builtin_fmaf(dt, gq, dA[i]);
                    sB = __builtin_fmaf(g, bb[j], sB);
                    vb[j] = g * w;
                    vc[j] = dy * hs[k][i];
                    if constexpr (HAS_Z) y = __builtin_fmaf(cc[j], hs[k][i], y);
                }
                swap_add32x4(vb, vc, wsum + 4 * q);
            }
            sB = sum_group<G>(sB);
            sq = sum_group<G>(sq);
            if constexpr (HAS_Z) y = sum_group<G>(y);
            const float du = __builtin_fmaf(dy, Dd, dt * sB);
            const float ddt = __builtin_fmaf(uu, sB, sq * kLn2);
            float ddl = ddt;
            if constexpr (SOFTPLUS) ddl *= sigmoid_f(dlv[k] + dbias);
            dD_acc = __builtin_fmaf(dy, uu, dD_acc);
            db_acc += live ? ddl : 0.0f;
            if (live && sub == 0) {
                const int so = tok_soff(t);
                buf_store_s<T>(du_rs, lane_off, so, du);
                buf_store_s<T>(dd_rs, lane_off, so, ddl);
                if constexpr (HAS_Z) {
                    const float yf = __builtin_fmaf(Dd, uu, y);
                    buf_store_s<T>(dz_rs, lane_off, so, dov[k] * yf * sgz * __builtin_fmaf(zv[k], 1.0f - sgz, 1.0f));
                }
            }
            // dB_t, dC_t: the wave's sums over its channels (lane sums, no LDS);
            // the 4 waves' sums meet in sp.
            const float tot = lane_sum_finish<V, G == 2>(wsum, lane);
            if ((lane & kWriter) == 0) {
                const int vi = (lane >> kSumShift) & (V - 1);
                const int h = G == 2 ? (lane & 1) : 0;
                const int n = vi < NL ? h * NL + vi : N + h * NL + (vi - NL);
                sp[(wave * kCk + k4 + k) * NOUT + n] = tot;
            }
#if MAMBA_BWD_TOKEN_BARRIER
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
    };

    {
        const int64_t s_last = t_begin + ((t_end - t_begin - 1) / kCk) * kCk;
        stage_block(s_last);
        fetch_ck(s_last);
    }
    const int64_t nwin = (t_end - t_begin + kWin - 1) / kWin;
    for (int64_t wi = nwin - 1; wi >= 0; --wi) {
        const int64_t w0 = t_begin + wi * kWin;
        starts = window_starts(ds_row, w0, t_end, lane, p.init != nullptr);
        __syncthreads();
        stage_rows<T, N, 2>(sBC, B_row, C_row, w0, t_end, tid);
        __syncthreads();
        const int64_t wend = (w0 + kWin < t_end) ? w0 + kWin : t_end;
        const int nblk16 = static_cast<int>((wend - w0 + kCk - 1) / kCk);
        for (int kb = nblk16 - 1; kb >= 0; --kb) {
            // 16-token block [s, s + 16): its checkpoint, the state before s + 8,
            // then its four pieces last to first (pieces past the chunk end are
            // identity steps and are skipped).
            const int64_t s = w0 + kb * kCk;
            const int os = kb * kCk;
            float* sp = sP[buf];
            float ck0[NL], ck8[NL];
            // The block's staged inputs and checkpoint have landed.
            s_cur = s;
            __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
            // dt of the block's tokens from the staged delta, with the aggregate
            // pass's arithmetic (bitwise the same values); the G lanes of a
            // channel take every G-th token.  Lanes of one wave read and write
            // LDS in order, so the other lanes see these rows when they load them.
            for (int k = lane % G; k < kCk; k += G)
                reinterpret_cast<float*>(stg)[k * CPW + chw] = step_size<SOFTPLUS>(stg_val(4, k), dbias);
            // local checkpoint + exp(A * sum dt) * (state entering the chunk)
            {
                const bool fresh = !carried_in || ck_flag != 0.0f;
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    ck0[i] = fresh ? ckv[i] : __builtin_fmaf(exp2_fast(Al2[i] * ck_cdt), hinv[i], ckv[i]);
            }
#pragma unroll
            for (int i = 0; i < NL; ++i) ck8[i] = ck0[i];
            advance4(ck8, s, os);
#if MAMBA_BWD_ST4_LDS
#pragma unroll
            for (int q = 0; q < NL / 4; ++q)
                sH4[q * kBlk + tid] = make_float4(ck8[4 * q], ck8[4 * q + 1], ck8[4 * q + 2], ck8[4 * q + 3]);
#endif
            advance4(ck8, s + 4, os + 4);
#pragma unroll
            for (int i = 0; i < NL; ++i) ck8[i] = opaque(ck8[i]);
            // Pieces last to first, one loop body (unrolling the four lets the
            // compiler interleave them and run out of registers).
#pragma unroll 1
            for (int j = kCk / kPiece - 1; j >= 0; --j) {
                const int64_t s4 = s + j * kPiece;
                if (s4 >= t_end) continue;                 // identity steps only
                float st[NL];
#pragma unroll
                for (int i = 0; i < NL; ++i) st[i] = j >= 2 ? ck8[i] : ck0[i];
#if MAMBA_BWD_ST4_LDS
                if (j == 1) {
#pragma unroll
                    for (int q = 0; q < NL / 4; ++q) {
                        const float4 v = sH4[q * kBlk + tid];
                        st[4 * q] = v.x; st[4 * q + 1] = v.y; st[4 * q + 2] = v.z; st[4 * q + 3] = v.w;
                    }
                } else if (j == 3) {
#else
                if (j & 1) {
#endif
                    advance4(st, s4 - kPiece, os + j * kPiece - kPiece);
#pragma unroll
                    for (int i = 0; i < NL; ++i) st[i] = opaque(st[i]);
                }
                piece(s4, os + j * kPiece, j * kPiece, st, sp);
            }
            __syncthreads();
            flush16(sp, s);
            buf ^= 1;
        }
    }

    if (!active) return;
    float* pw = p.part_w + (b * p.nchunks + c) * (N + 2) * p.dim + d;
#pragma unroll
    for (int i = 0; i < NL; ++i) pw[static_cast<int64_t>(n0 + i) * p.dim] = dA[i];
    if (sub == 0) {
        pw[static_cast<int64_t>(N) * p.dim] = dD_acc;
        pw[static_cast<int64_t>(N + 1) * p.dim] = db_acc;
    }
}

// 5a. dB[b, t, n] and dC[b, t, n]: sums of the per-block partials, in block order.
template <typename T, int N>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part, void* dB, void* dC,
                                                            int64_t rows, int nblk) {
    constexpr int V = 2 * N;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= rows * V) return;
    const int64_t row = e / V;
    const int j = static_cast<int>(e % V);
    const float* src = part + row * nblk * V + j;
    float s = 0.0f;
    for (int k = 0; k < nblk; ++k) s += src[static_cast<int64_t>(k) * V];
    if (j < N) Elem<T>::store(dB, row * N + j, s);
    else Elem<T>::store(dC, row * N + j - N, s);
}

// 5b. dA (D, N), dD (D,), ddelta_bias (D,): sums over rows and chunks.  A block
// covers 64 outputs with 4 threads each; thread g sums the parts g, g + 4, ...
// (two accumulators), then the 4 partial sums are added in a fixed order.
template <int N>
__global__ __launch_bounds__(256) void bwd_reduce_w_kernel(const float* __restrict__ part, float* dA, float* dD,
                                                           float* dbias, int64_t nparts, int dim) {
    __shared__ float red[4][64];
    const int64_t nout = static_cast<int64_t>(N + 2) * dim;
    const int lane = threadIdx.x & 63;
    const int grp = threadIdx.x >> 6;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    float s0 = 0.0f, s1 = 0.0f;
    if (e < nout) {
        const float* src = part + e;
        int64_t i = grp;
        for (; i + 4 < nparts; i += 8) {
            s0 += src[i * nout];
            s1 += src[(i + 4) * nout];
        }
        if (i < nparts) s0 += src[i * nout];
    }
    red[grp][lane] = s0 + s1;
    __syncthreads();
    if (grp != 0 || e >= nout) return;
    const float s = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    const int k = static_cast<int>(e / dim);
    const int d = static_cast<int>(e % dim);
    if (k < N) dA[static_cast<int64_t>(d) * N + k] = s;
    else if (k == N) { if (dD) dD[d] = s; }
    else if (dbias) dbias[d] = s;
}

// Lanes per channel in the main pass.
constexpr int lanes_per_channel(int64_t n) { return n == 16 ? MAMBA_BWD_G16 : (n == 8 ? MAMBA_BWD_G8 : 1); }

// Workspace layout (byte offsets, each region 256-byte aligned).
struct BwdLayout {
    size_t h_carry, h_agg, g_carry, p_rev, ckpt, part_bc, part_w, x0, r0, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, const ScanPlan& plan) {
    const size_t count = static_cast<size_t>(batch * dim * dstate);
    const size_t slots = plan.nchunks > 1 ? static_cast<size_t>(plan.nchunks - 1) : 0;
    const size_t carry = align256(slots * count * sizeof(float));
    const int64_t nk = (seqlen + kCk - 1) / kCk;
    const int64_t cpb = kBlk / lanes_per_channel(dstate);
    const int64_t nblk = (dim + cpb - 1) / cpb;
    BwdLayout l;
    l.h_carry = 0;
    l.h_agg = l.h_carry + carry;
    l.g_carry = l.h_agg + carry;
    l.p_rev = l.g_carry + carry;
    l.ckpt = l.p_rev + carry;
    l.part_bc = l.ckpt + align256(static_cast<size_t>(batch * nk * (dstate + 2) * dim) * sizeof(float));
    l.part_w = l.part_bc + align256(static_cast<size_t>(batch * seqlen * nblk * 2 * dstate) * sizeof(float));
    l.x0 = l.part_w + align256(static_cast<size_t>(batch * plan.nchunks * (dstate + 2) * dim) * sizeof(float));
    l.r0 = l.x0 + align256(count * sizeof(float));
    l.total = l.r0 + align256(count * sizeof(float));
    return l;
}

template <typename T, int N>
hipError_t launch_bwd_typed(const ScanBwdArgs& a, const ScanPlan& plan, const BwdLayout& l) {
    char* ws = static_cast<char*>(a.ws);
    BwdKParams p{};
    p.u = a.u; p.delta = a.delta; p.A = a.A; p.B = a.B; p.C = a.C; p.D = a.D; p.z = a.z;
    p.delta_bias = a.delta_bias; p.doc_start = a.doc_start; p.dout = a.dout;
    p.h_agg_P = reinterpret_cast<float*>(ws + l.h_carry);
    p.h_agg_H = reinterpret_cast<float*>(ws + l.h_agg);
    p.ckpt_out = reinterpret_cast<float*>(ws + l.ckpt);
    p.h_carry = reinterpret_cast<const float*>(ws + l.h_carry);
    p.g_carry = reinterpret_cast<float*>(ws + l.g_carry);
    p.p_rev = reinterpret_cast<float*>(ws + l.p_rev);
    p.ckpt = reinterpret_cast<const float*>(ws + l.ckpt);
    p.part_bc = reinterpret_cast<float*>(ws + l.part_bc);
    p.part_w = reinterpret_cast<float*>(ws + l.part_w);
    p.du = a.du; p.ddelta = a.ddelta; p.dz = a.dz;
    p.init = a.initial_state;
    p.d_final = a.d_final_state;
    if (a.d_initial_state != nullptr) {
        p.x0 = reinterpret_cast<float*>(ws + l.x0);
        p.r0 = reinterpret_cast<float*>(ws + l.r0);
    }
    p.seqlen = a.seqlen;
    p.chunk_len = plan.chunk_len;
    p.nchunks = plan.nchunks;
    p.nslots = plan.nchunks - 1;
    p.nk = (a.seqlen + kCk - 1) / kCk;
    p.dim = static_cast<int>(a.dim);
    p.nbatch = static_cast<int>(a.batch);
    constexpr int G = lanes_per_channel(N);
    constexpr int CPB = kBlk / G;
    p.nblk = static_cast<int>((a.dim + CPB - 1) / CPB);
    const unsigned gx = static_cast<unsigned>((a.dim + kBlk - 1) / kBlk);
    const int64_t count = a.batch * a.dim * N;

    dim3 g1(gx, static_cast<unsigned>(plan.nchunks), static_cast<unsigned>(a.batch));
    if (a.z) {
        if (a.softplus) hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, true, true>), g1, dim3(kBlk), 0, a.stream, p);
        else hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, true, false>), g1, dim3(kBlk), 0, a.stream, p);
    } else {
        if (a.softplus) hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, false, true>), g1, dim3(kBlk), 0, a.stream, p);
        else hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, false, false>), g1, dim3(kBlk), 0, a.stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gc(static_cast<unsigned>((count + 255) / 256));
    if (p.nslots > 0) {
        hipLaunchKernelGGL(bwd_fwd_carry_kernel, gc, dim3(256), 0, a.stream, p.h_agg_P,
                           static_cast<const float*>(p.h_agg_H), a.initial_state, count, p.nslots);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.nslots > 0 || a.d_initial_state != nullptr) {
        hipLaunchKernelGGL(bwd_rev_carry_kernel, gc, dim3(256), 0, a.stream, p.g_carry, static_cast<const float*>(p.p_rev),
                           a.d_final_state, static_cast<const float*>(p.x0), static_cast<const float*>(p.r0),
                           a.d_initial_state, count, p.nslots);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 g4(static_cast<unsigned>(p.nblk), static_cast<unsigned>(plan.nchunks), static_cast<unsigned>(a.batch));
    if (a.z) {
        if (a.softplus) hipLaunchKernelGGL((bwd_chunk_kernel<T, N, G, true, true>), g4, dim3(kBlk), 0, a.stream, p);
        else hipLaunchKernelGGL((bwd_chunk_kernel<T, N, G, true, false>), g4, dim3(kBlk), 0, a.stream, p);
    } else {
        if (a.softplus) hipLaunchKernelGGL((bwd_chunk_kernel<T, N, G, false, true>), g4, dim3(kBlk), 0, a.stream, p);
        else hipLaunchKernelGGL((bwd_chunk_kernel<T, N, G, false, false>), g4, dim3(kBlk), 0, a.stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = a.batch * a.seqlen;
    hipLaunchKernelGGL((bwd_reduce_bc_kernel<T, N>), dim3(static_cast<unsigned>((rows * 2 * N + 255) / 256)),
                       dim3(256), 0, a.stream, static_cast<const float*>(p.part_bc), a.dB, a.dC, rows, p.nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_reduce_w_kernel<N>), dim3(static_cast<unsigned>(((N + 2) * a.dim + 63) / 64)),
                       dim3(256), 0, a.stream, static_cast<const float*>(p.part_w), a.dA, a.dD, a.ddelta_bias,
                       a.batch * plan.nchunks, p.dim);
    return hipGetLastError();
}

}  // namespace

int64_t scan_bwd_kernel_dstate(int64_t dstate, int nheads) {
    if (nheads != 0 || dstate < 1) return 0;
    return dstate <= 4 ? 4 : dstate <= 8 ? 8 : dstate <= 16 ? 16 : 0;
}

bool scan_bwd_supported(int64_t dstate, int nheads) { return scan_bwd_kernel_dstate(dstate, nheads) != 0; }

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool bf16) {
    (void)bf16;   // the layout holds float32 carries, checkpoints and partials for either I/O dtype
    return bwd_layout(batch, seqlen, dim, dstate, plan_scan(batch, seqlen, dim)).total;
}

hipError_t launch_selective_scan_bwd(const ScanBwdArgs& a) {
    const ScanPlan plan = plan_scan(a.batch, a.seqlen, a.dim);
    const BwdLayout l = bwd_layout(a.batch, a.seqlen, a.dim, a.dstate, plan);
    switch (a.dstate) {
        case 4: return a.bf16 ? launch_bwd_typed<bf16_t, 4>(a, plan, l) : launch_bwd_typed<float, 4>(a, plan, l);
        case 8: return a.bf16 ? launch_bwd_typed<bf16_t, 8>(a, plan, l) : launch_bwd_typed<float, 8>(a, plan, l);
        case 16: return a.bf16 ? launch_bwd_typed<bf16_t, 16>(a, plan, l) : launch_bwd_typed<float, 16>(a, plan, l);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mamba
