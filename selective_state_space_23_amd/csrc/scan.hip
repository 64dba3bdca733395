// Selective-scan forward over packed documents, gfx950.
//
// What it computes (Mamba skill page: S6 block diagram, "Core Concept", the S6
// code and the "Mamba-2 (SSD)" section; axolotl page: per-document restart):
//   dt_t  = softplus(delta_t + delta_bias)          (or without softplus)
//   h_t   = exp(dt_t * A) * h_{t-1} + dt_t * u_t * B_t   per channel d, state n
//   y_t   = C_t . h_t + D * u_t,   out_t = y_t * silu(z_t)
//   h := 0 at every document start; final_state = h after the last token.
// A is (D, N) (diagonal per channel) or (H,) (one scalar per head).
//
// Mapping ("lanes are channels").  One lane owns one channel d of one row b and
// keeps its N states in fp32 VGPRs; the 64 lanes of a wave are 64 consecutive
// channels, so every activation load and store of a wave is one contiguous 128 B
// (bf16) span of a (B, L, D) row.  B_t and C_t, shared by all channels, are
// staged per 64-token window in LDS as fp32 and read back with broadcast 16-byte
// loads; doc_start becomes a wave-uniform bit mask per window, and a document
// start rides in the decay's exponent (-inf).  Per element the recurrence costs
// one v_exp_f32 and four fp32 ops (dt*A, dt*u*B, the state FMA, the C*h FMA).
// With scalar-A heads the states of a channel share one decay per token, so
// N / 16 consecutive lanes split them (16 each) and add their parts of C . h.
//
// Parallelism along L.  B * D / 64 waves are far too few to fill 256 CUs at the
// target shapes, so L is cut into chunks and the chunks are joined with the
// associative operator of the "Hardware-Aware Parallel Scan" section:
//   pass 1 (aggregate): each chunk runs its recurrence from a zero state and
//          stores (P, H): P = prod of exp(dt A) over the chunk (0 if a document
//          starts inside it), H = its end state (the last chunk's is never
//          needed; the tokens before a chunk's last document start cannot reach
//          it).  With per-channel A it also hands the step sizes dt to pass 3
//          and, in the fused call, forms u from x (storing it when asked to).
//   pass 2 (carry):     per (b, d, n), carry_{c+1} = P_c * carry_c + H_c.
//   pass 3 (output):    every chunk reruns its recurrence from its carry and
//          writes out and, for the last chunk, final_state.
// The (B, L, D, N) state trajectory is never stored.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

constexpr int kScanBlock = 256;    // 4 independent waves, 256 consecutive channels
#ifndef MAMBA_SCAN_SCHED_BARRIER
#define MAMBA_SCAN_SCHED_BARRIER 1
#endif
#ifndef MAMBA_SCAN_GROUP
#define MAMBA_SCAN_GROUP 4
#endif
#ifndef MAMBA_SCAN_TARGET_WAVES
#define MAMBA_SCAN_TARGET_WAVES 4096
#endif
#ifndef MAMBA_SCAN_WAVES_PER_EU
#define MAMBA_SCAN_WAVES_PER_EU 4
#endif
constexpr int kGroup = MAMBA_SCAN_GROUP;   // tokens whose activations are fetched together
constexpr int kNoStore = 0x7fffff00;       // buffer offset past any resource: the access is dropped
// The fused conv of the per-channel scan (template argument CONV).
constexpr int kConvNone = 0;               // the activations loaded are u
constexpr int kConvStoreU = 1;             // loaded x, u formed and stored (pass 1)
constexpr int kConvNoStore = 2;            // loaded x, u formed, not stored

struct ScanKParams {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* delta_bias;
    const uint8_t* doc_start;
    const float* initial_state;   // (B, D, N) or null: state before token 0
    void* out;
    float* final_state;
    float* ws_P;        // [nchunks-1][B][D][N]: pass 1 P, then pass 2 carries
    float* ws_H;        // [nchunks-1][B][D][N]: pass 1 H
    const void* conv_x;       // fused conv (pass 1): its input x (B, L, D)
    const float* conv_w;      // (D, 4)
    const float* conv_b;      // (D,) or null
    const void* conv_state;   // (B, D, 3) or null
    void* u_out;              // (B, L, D): pass 1 stores u here
    void* dt_ws;              // (B, L, D), I/O dtype: step sizes from pass 1 for pass 3 (per-channel A)
    int64_t nslots;           // chunks with an aggregate slot (nchunks - 1)
    int64_t seqlen;
    int64_t chunk_len;
    int dim;
    int nheads;
    int headdim;
    int nbatch;
    int softplus;
};

// Raw buffer access: a 128-bit resource (base, size) held in SGPRs plus a 32-bit
// per-lane byte offset, so addresses need no 64-bit VALU arithmetic.
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

template <typename T>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t rs, int byte_off, float v) {
    if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rs, byte_off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, byte_off, 0, 0);
}

// The same with the offset split into a lane part (channel) and a wave-uniform
// part (token) that rides in the instruction's scalar offset: no per-token VALU
// address arithmetic.
template <typename T>
__device__ __forceinline__ float buf_load_s(__amdgpu_buffer_rsrc_t rs, int lane_off, int tok_off) {
    if constexpr (sizeof(T) == 2) {
        const uint16_t v = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, lane_off, tok_off, 0));
        return bf16_to_f32(v);
    } else {
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, lane_off, tok_off, 0)));
    }
}

template <typename T>
__device__ __forceinline__ void buf_store_s(__amdgpu_buffer_rsrc_t rs, int lane_off, int tok_off, float v) {
    if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), rs, lane_off, tok_off, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, lane_off, tok_off, 0);
}

// OUTPUT = false: pass 1 (aggregate of one chunk from a zero state).
// OUTPUT = true:  pass 3 (outputs of one chunk from its carried state).
//
// Data movement inside a chunk:
//   - B_t (and C_t) are shared by all channels: the block stages them for a
//     64-token window in LDS as fp32 (one coalesced 16-byte load per thread,
//     converted once for the 256 channels of the block), and every wave reads
//     them back with broadcast ds_read_b128, so each lane gets B_t[n..n+3] as
//     VGPR operands with no per-lane conversion;
//   - per-lane activations (u, delta, z) of the next group of G tokens are
//     fetched while the current group computes: two register sets in ping-pong,
//     so no loaded register is ever copied (a copy would wait on the load);
//   - addresses are a wave-uniform 64-bit row base plus a 32-bit element offset.
//
// CONV (per-channel A): the activations loaded are the conv input x, and each
// lane forms u = SiLU(bias + w . (x[t-3], x[t-2], x[t-1], x[t])) itself from a
// 3-token history in registers (cleared at document starts, primed from the
// tokens before the chunk), rounded to T, and scans with it.  kConvStoreU (pass
// 1): u is also stored, for pass 3 and the caller.  kConvNoStore: not stored
// (the caller asked for no u); pass 3 then forms u again the same way.  The
// arithmetic and its order are those of the standalone conv kernel, so u is
// bitwise the same in every pass.
//
// DTWS (per-channel A): pass 1 stores dt (rounded to T) in the workspace and
// pass 3 reads it back instead of recomputing the softplus; without it pass 3
// recomputes dt from delta and the workspace holds the carries only.
template <typename T, int N, bool HEADS, bool OUTPUT, bool HAS_Z, bool SOFTPLUS, int CONV, bool DTWS>
__global__ __launch_bounds__(kScanBlock) __attribute__((amdgpu_waves_per_eu(MAMBA_SCAN_WAVES_PER_EU))) void scan_chunk_kernel(
    const ScanKParams p) {
    static_assert(CONV == kConvNone || !HEADS, "the conv is fused for per-channel A");
    static_assert(!(OUTPUT && CONV == kConvStoreU), "u is stored by pass 1");
    static_assert(!(HEADS && DTWS), "step sizes are handed over for per-channel A only");
    constexpr int G = kGroup;
    constexpr int kRows = OUTPUT ? 2 : 1;                      // B and C, or B only
    // Tokens per staged window: 64, or 32 where 64 tokens of B and C in fp32
    // would take over 32 KB of LDS (N = 128: 64 KB held the output pass of fp32
    // scalar-A heads to two workgroups a CU).  A power of two up to 64: the
    // window's document starts are one wave-wide bit mask.
    constexpr int kWin = kRows * 64 * N * 4 > 32768 ? 32 : 64;
    static_assert(kWin == 32 || kWin == 64, "window of at most one bit per lane");
    constexpr int kWinFloats = kWin * N;                       // one tensor's window
    __shared__ float4 smem4[kRows * kWinFloats / 4];
    float* smem = reinterpret_cast<float*>(smem4);

    // Scalar-A heads: the N states of a channel share one decay per token, so
    // LPC lanes split them (NL = 16 each) and add their parts of C . h with DPP;
    // per-channel A keeps all N states of a channel in one lane.
    constexpr int LPC = (HEADS && N > 16) ? N / 16 : 1;
    constexpr int NL = N / LPC;
    static_assert(LPC == 1 || LPC == 2 || LPC == 4 || LPC == 8, "lane groups inside a DPP row half");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int d = (blockIdx.x * kScanBlock + tid) / LPC;      // channel
    const int n0 = (tid % LPC) * NL;                          // this lane's first state
    const bool active = d < p.dim;
    const int dc = active ? d : p.dim - 1;          // clamped channel for loads
    const int64_t c = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t L = p.seqlen;
    const int64_t t_begin = c * p.chunk_len;
    const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;
    const int head = HEADS ? dc / p.headdim : 0;
    const int nd = HEADS ? p.nheads : p.dim;        // width of delta rows
    const int dsel = HEADS ? head : dc;

    // Per-row buffer resources (wave-uniform base + size) and 32-bit byte offsets
    // for the per-lane activations: t * width + channel fits in 31 bits.
    constexpr int kEsz = static_cast<int>(sizeof(T));
    const int64_t act_row = L * p.dim;
    const __amdgpu_buffer_rsrc_t u_rs =
        make_rsrc(static_cast<const T*>(CONV != kConvNone ? p.conv_x : p.u) + b * act_row, act_row * kEsz);
    const __amdgpu_buffer_rsrc_t uo_rs =
        make_rsrc(static_cast<T*>(CONV == kConvStoreU ? p.u_out : p.out) + b * act_row, act_row * kEsz);
    // With the hand-off both passes use the same rounded dt.
    constexpr bool kDtWs = DTWS;
    const __amdgpu_buffer_rsrc_t dl_rs =
        make_rsrc(static_cast<const T*>((kDtWs && OUTPUT) ? p.dt_ws : p.delta) + b * L * nd, L * nd * kEsz);
    const __amdgpu_buffer_rsrc_t dto_rs =
        make_rsrc(static_cast<T*>(kDtWs ? p.dt_ws : p.out) + b * act_row, kDtWs ? act_row * kEsz : 0);
    const __amdgpu_buffer_rsrc_t z_rs =
        make_rsrc(static_cast<const T*>(HAS_Z ? p.z : (CONV != kConvNone ? p.conv_x : p.u)) + b * act_row,
                  HAS_Z ? act_row * kEsz : 0);
    const T* B_row = static_cast<const T*>(p.B) + b * L * N;
    const T* C_row = static_cast<const T*>(p.C) + b * L * N;
    const uint8_t* ds_row = p.doc_start ? p.doc_start + b * L : nullptr;

    // Per-channel constants: A scaled by log2(e) so exp(dt A) = exp2(dt * Al2).
    float Al2[HEADS ? 1 : N];
    if constexpr (HEADS) {
        Al2[0] = p.A[head] * kLog2e;
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) Al2[n] = p.A[static_cast<int64_t>(dc) * N + n] * kLog2e;
    }
    const float dbias = p.delta_bias ? p.delta_bias[dsel] : 0.0f;
    const float Dd = (OUTPUT && p.D) ? p.D[dc] : 0.0f;

    // Chunk carry (pass 3) or zero.
    const int64_t slot_stride = static_cast<int64_t>(p.nbatch) * p.dim * N;
    const int64_t my_slot = (b * p.dim + dc) * N + n0;
    float h[NL];
    if (OUTPUT && (c > 0 || p.initial_state != nullptr)) {
        const float* carry = c > 0 ? p.ws_P + (c - 1) * slot_stride + my_slot : p.initial_state + my_slot;
#pragma unroll
        for (int n = 0; n < NL; ++n) h[n] = carry[n];
    } else {
#pragma unroll
        for (int n = 0; n < NL; ++n) h[n] = 0.0f;
    }
    float sum_dt = 0.0f;          // pass 1: sum of dt since the chunk start
    bool any_reset = false;       // pass 1: a document starts inside the chunk

    // Fused conv: weights and the input history x[t-1], x[t-2], x[t-3] as seen by
    // the chunk's first token (taps before its document start read zero).
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f, xh1 = 0.0f, xh2 = 0.0f, xh3 = 0.0f;
    // Token 0 continues the conv history although the scan restarts there: a
    // conv_state without an initial_state.
    bool conv_keep0 = false;
    if constexpr (CONV != kConvNone) {
        conv_keep0 = p.conv_state != nullptr && !(ds_row != nullptr && ds_row[0] != 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[j] = p.conv_w[static_cast<int64_t>(dc) * 4 + j];
        cb = p.conv_b ? p.conv_b[dc] : 0.0f;
        auto hist = [&](int k) -> float {              // x[t_begin - k]
            const int64_t t = t_begin - k;
            if (t >= 0) return buf_load<T>(u_rs, static_cast<int>((t * p.dim + dc) * kEsz));
            if (p.conv_state == nullptr) return 0.0f;
            return Elem<T>::load(p.conv_state, (b * p.dim + dc) * 3 + (3 - k));
        };
        // The conv's own rule for token 0: it starts a document unless a
        // history is given (the scan's rule looks at initial_state instead).
        auto starts_at = [&](int64_t t) -> bool {
            if (t < 0) return false;
            return (t == 0 && p.conv_state == nullptr) || (ds_row != nullptr && ds_row[t] != 0);
        };
        const bool s1 = starts_at(t_begin - 1), s2 = starts_at(t_begin - 2);
        xh1 = hist(1);
        xh2 = s1 ? 0.0f : hist(2);
        xh3 = (s1 || s2) ? 0.0f : hist(3);
    }

    auto load_group = [&](int64_t g0, float (&uu)[G], float (&dl)[G], float (&zz)[G]) {
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = static_cast<int>((g0 + k < t_end) ? g0 + k : t_end - 1);  // clamp the tail
            uu[k] = buf_load_s<T>(u_rs, dc * kEsz, t * p.dim * kEsz);
            dl[k] = buf_load_s<T>(dl_rs, dsel * kEsz, t * nd * kEsz);
            if constexpr (OUTPUT && HAS_Z) zz[k] = buf_load_s<T>(z_rs, dc * kEsz, t * p.dim * kEsz);
            else zz[k] = 0.0f;
        }
    };

    // Stage B (and C) of tokens w0 .. w0+63 into LDS as fp32.  Each step moves
    // VW consecutive elements of one token row (16 bytes when the row allows);
    // tokens past the chunk end are clamped to its last token and never read back.
    auto stage_window = [&](int64_t w0) {
        constexpr int kVecElems = 16 / static_cast<int>(sizeof(T));
        constexpr int VW = N < kVecElems ? N : kVecElems;
        constexpr int kStepsPerTensor = kWinFloats / VW;
        for (int i = tid; i < kRows * kStepsPerTensor; i += kScanBlock) {
            const int tensor = i / kStepsPerTensor;
            const int e0 = (i % kStepsPerTensor) * VW;        // element index inside the window
            const int tok = e0 / N;
            const int n0 = e0 % N;
            const int64_t t = (w0 + tok < t_end) ? w0 + tok : t_end - 1;
            const T* src = (tensor == 0 ? B_row : C_row) + t * N + n0;
            float* dst = smem + tensor * kWinFloats + e0;
            float v[VW];
            if constexpr (sizeof(T) == 2) {
                uint32_t wv[VW / 2];
                if constexpr (VW == 8) {
                    const uint4 r = *reinterpret_cast<const uint4*>(src);
                    wv[0] = r.x; wv[1] = r.y; wv[2] = r.z; wv[3] = r.w;
                } else if constexpr (VW == 4) {
                    const uint2 r = *reinterpret_cast<const uint2*>(src);
                    wv[0] = r.x; wv[1] = r.y;
                } else {
                    wv[0] = *reinterpret_cast<const uint32_t*>(src);
                }
#pragma unroll
                for (int k = 0; k < VW / 2; ++k) {
                    v[2 * k] = __uint_as_float(wv[k] << 16);
                    v[2 * k + 1] = __uint_as_float(wv[k] & 0xffff0000u);
                }
            } else {
                const float4 r = *reinterpret_cast<const float4*>(src);
                v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
            }
#pragma unroll
            for (int k = 0; k < VW; k += 4)
                *reinterpret_cast<float4*>(dst + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
        }
    };

    uint64_t starts = 0;
    // Pass 1: the first token whose recurrence reaches the chunk's aggregate.  The
    // state restarts from zero at the chunk's last document start, so the
    // tokens before it only need their u and dt (stored for pass 3); the last
    // chunk's aggregate is never used at all.  Uniform over the block.
    int64_t rec_from = t_begin;
    if constexpr (!OUTPUT) {
        if (c >= p.nslots) {
            rec_from = t_end;
        } else {
            for (int64_t w0 = t_begin; w0 < t_end; w0 += kWin) {
                const int64_t tl = w0 + lane;
                const bool st = lane < kWin && tl < t_end &&
                                ((tl == 0 && p.initial_state == nullptr) || (ds_row != nullptr && ds_row[tl] != 0));
                const uint64_t m = __ballot(st);
                if (m != 0) rec_from = w0 + 63 - __builtin_clzll(m);
            }
        }
    }
    // FAST: every token of the group is inside the chunk and none starts a
    // document (wave-uniform; all but a few groups), so the masks below fold
    // away and stores go to the clamped channel (an inactive lane writes the
    // value its clamped channel's own lane writes) with the token in the scalar
    // offset.  REC (always, in pass 3): the group runs the recurrence; pass 1's
    // groups before rec_from only form u and dt.
    auto compute_group = [&](auto fast_tag, auto rec_tag, int64_t g0, float (&cu)[G], const float (&cd)[G],
                             const float (&cz)[G]) {
        constexpr bool FAST = decltype(fast_tag)::value;
        constexpr bool REC = OUTPUT || decltype(rec_tag)::value;
        const int off = static_cast<int>((g0 - t_begin) & (kWin - 1));
        // Phase 1: the per-token inputs of the recurrence for the whole group
        // (dt, and w = dt u; the conv, softplus and their stores in pass 1).
        // These are long dependent chains (exp, log, rcp); the
        // group's tokens are independent here, so their chains overlap instead
        // of stalling each token's state updates.
        float dtk[G], wk[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            // Tokens past the chunk end run as identity steps (dt = 0: decay 1, no
            // input) so the group stays straight-line code.
            const bool valid = FAST || g0 + k < t_end;
            const int64_t t = g0 + k;
            const bool reset = !FAST && ((starts >> (off + k)) & 1ull);
            float dt;
            if constexpr (kDtWs && OUTPUT) {
                dt = cd[k];                                   // stored by pass 1
            } else {
                dt = cd[k] + dbias;
                if constexpr (SOFTPLUS) dt = softplus_f(dt);
                if constexpr (kDtWs) {
                    if constexpr (sizeof(T) == 2) dt = bf16_to_f32(f32_to_bf16(dt));
                    if constexpr (FAST) buf_store_s<T>(dto_rs, dc * kEsz, static_cast<int>(t) * p.dim * kEsz, dt);
                    else buf_store<T>(dto_rs, (active && valid) ? (static_cast<int>(t) * p.dim + d) * kEsz : kNoStore, dt);
                }
            }
            dt = valid ? dt : 0.0f;
            if constexpr (!OUTPUT && REC) {
                any_reset = any_reset || reset;
                sum_dt = (reset ? 0.0f : sum_dt) + dt;
            }
            float uk = cu[k];
            if constexpr (CONV != kConvNone) {
                const float xt = cu[k];
                const bool creset = reset && !(t == 0 && conv_keep0);
                xh1 = creset ? 0.0f : xh1;
                xh2 = creset ? 0.0f : xh2;
                xh3 = creset ? 0.0f : xh3;
                float acc = __builtin_fmaf(cw[3], xt, cb);
                acc = __builtin_fmaf(cw[2], xh1, acc);
                acc = __builtin_fmaf(cw[1], xh2, acc);
                acc = __builtin_fmaf(cw[0], xh3, acc);
                uk = silu_f(acc);
                if constexpr (sizeof(T) == 2) uk = bf16_to_f32(f32_to_bf16(uk));   // u as stored
                // Branchless: a store past the resource's end is dropped by the
                // hardware, and a branch here would double the register footprint.
                if constexpr (CONV == kConvStoreU) {
                    if constexpr (FAST) buf_store_s<T>(uo_rs, dc * kEsz, static_cast<int>(t) * p.dim * kEsz, uk);
                    else buf_store<T>(uo_rs, (active && valid) ? (static_cast<int>(t) * p.dim + d) * kEsz : kNoStore, uk);
                }
                xh3 = xh2;
                xh2 = xh1;
                xh1 = xt;
            }
            dtk[k] = dt;
            wk[k] = dt * uk;
            if constexpr (CONV != kConvNone) cu[k] = uk;     // x is not needed past this point
        }
        if constexpr (!REC) return;
        // Phase 2: the recurrence, token by token.
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const bool valid = FAST || g0 + k < t_end;
            const int64_t t = g0 + k;
            // A document start multiplies the carried state by exp2(-inf) = 0: the
            // reset rides in the exponent's addend, with no branch and no extra op.
            const bool reset = !FAST && ((starts >> (off + k)) & 1ull);
            const float r = reset ? -__builtin_inff() : 0.0f;
            const float dt = dtk[k];
            const float w = wk[k];
            float y0 = 0.0f, y1 = 0.0f;          // two partial sums of C . h
            float a_head = 0.0f;
            if constexpr (HEADS) a_head = exp2_fast(__builtin_fmaf(dt, Al2[0], r));
            const float4* Bq = reinterpret_cast<const float4*>(smem + (off + k) * N + n0);
            const float4* Cq = reinterpret_cast<const float4*>(smem + kWinFloats + (off + k) * N + n0);
#pragma unroll
            for (int q = 0; q < NL / 4; ++q) {
                const float4 bv = Bq[q];
                float4 cv;
                if constexpr (OUTPUT) cv = Cq[q];
                const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
                const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = 4 * q + j;
                    float a;
                    if constexpr (HEADS) a = a_head;
                    else a = exp2_fast(__builtin_fmaf(dt, Al2[n], r));
                    h[n] = __builtin_fmaf(a, h[n], w * bb[j]);
                    if constexpr (OUTPUT) {
                        if (j == 0 || j == 2) y0 = __builtin_fmaf(cc[j], h[n], y0);
                        else y1 = __builtin_fmaf(cc[j], h[n], y1);
                    }
                }
            }
            if constexpr (OUTPUT) {
                float yp = y0 + y1;
                if constexpr (LPC > 1) yp = lane_group_sum<LPC>(yp);   // C . h over the channel's lanes
                float y = yp + Dd * cu[k];
                if constexpr (HAS_Z) y *= silu_f(cz[k]);
                if constexpr (FAST) buf_store_s<T>(uo_rs, dc * kEsz, static_cast<int>(t) * p.dim * kEsz, y);
                else if (active && valid) buf_store<T>(uo_rs, (static_cast<int>(t) * p.dim + d) * kEsz, y);
            }
            // Keep the scheduler from hoisting later tokens' exponentials: one
            // token already offers N independent chains, and hoisting only
            // raises register pressure.
#if MAMBA_SCAN_SCHED_BARRIER
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
    };

    float au[G], ad[G], az[G], bu[G], bd[G], bz[G];
    load_group(t_begin, au, ad, az);
    for (int64_t w0 = t_begin; w0 < t_end; w0 += kWin) {
        // Document starts of the window as a wave-uniform bit mask.
        {
            const int64_t tl = w0 + lane;
            bool st = false;
            // Token 0 starts a document unless the row continues an initial state.
            if (lane < kWin && tl < t_end)
                st = (tl == 0 && p.initial_state == nullptr) || (ds_row != nullptr && ds_row[tl] != 0);
            starts = __ballot(st);
        }
        if (OUTPUT || w0 + kWin > rec_from) {    // B is read by some group of the window
            __syncthreads();             // every wave is done with the previous window
            stage_window(w0);
            __syncthreads();
        }
        const int64_t wend = (w0 + kWin < t_end) ? w0 + kWin : t_end;
        auto run_group = [&](int64_t g0, float (&cu)[G], const float (&cd)[G], const float (&cz)[G]) {
            const int off = static_cast<int>((g0 - t_begin) & (kWin - 1));
            const bool fast = g0 + G <= t_end && ((starts >> off) & ((1ull << G) - 1)) == 0;
            if (!OUTPUT && g0 + G <= rec_from) {
                if constexpr (!OUTPUT) {
                    if (fast) compute_group(std::true_type{}, std::false_type{}, g0, cu, cd, cz);
                    else compute_group(std::false_type{}, std::false_type{}, g0, cu, cd, cz);
                }
            } else if (fast) {
                compute_group(std::true_type{}, std::true_type{}, g0, cu, cd, cz);
            } else {
                compute_group(std::false_type{}, std::true_type{}, g0, cu, cd, cz);
            }
        };
        for (int64_t g0 = w0; g0 < wend; g0 += 2 * G) {
            load_group(g0 + G, bu, bd, bz);
            run_group(g0, au, ad, az);
            load_group(g0 + 2 * G, au, ad, az);
            run_group(g0 + G, bu, bd, bz);
        }
    }

    if (!active) return;
    if (OUTPUT) {
        if (p.final_state != nullptr && t_end == L) {
            float* fs = p.final_state + my_slot;
#pragma unroll
            for (int n = 0; n < NL; ++n) fs[n] = h[n];
        }
    } else {
        if (c >= p.nslots) return;          // the last chunk's aggregate is never used
        float* P = p.ws_P + c * slot_stride + my_slot;
        float* H = p.ws_H + c * slot_stride + my_slot;
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            float al;
            if constexpr (HEADS) al = Al2[0];
            else al = Al2[n];
            P[n] = any_reset ? 0.0f : exp2_fast(sum_dt * al);
            H[n] = h[n];
        }
    }
}

// Pass 2: carry_{c+1} = P_c * carry_c + H_c for every (b, d, n), written over
// ws_P[c] (ws_P[c] then holds the state entering chunk c + 1); carry_0 is the
// initial state (or zero).
__global__ __launch_bounds__(256) void scan_carry_kernel(float* __restrict__ ws_P, const float* __restrict__ ws_H,
                                                         const float* __restrict__ init, int64_t count,
                                                         int64_t nslots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= count) return;
    float carry = init != nullptr ? init[i] : 0.0f;
    // The chain over chunks is sequential; its loads are issued 16 chunks at a
    // time so that their latency overlaps.
    constexpr int kBatch = 16;
    int64_t c = 0;
    for (; c + kBatch <= nslots; c += kBatch) {
        float P[kBatch], H[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            P[k] = ws_P[(c + k) * count + i];
            H[k] = ws_H[(c + k) * count + i];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            carry = __builtin_fmaf(P[k], carry, H[k]);
            ws_P[(c + k) * count + i] = carry;
        }
    }
    for (; c < nslots; ++c) {
        carry = __builtin_fmaf(ws_P[c * count + i], carry, ws_H[c * count + i]);
        ws_P[c * count + i] = carry;
    }
}

// Byte offset of the step-size array in the per-channel scan's workspace: after
// the two carry arrays, rounded up to 256 bytes.
size_t dt_ws_offset(int64_t batch, int64_t dim, int64_t dstate, const ScanPlan& plan) {
    const size_t carries =
        plan.nchunks > 1
            ? static_cast<size_t>(2 * (plan.nchunks - 1)) * static_cast<size_t>(batch * dim * dstate) * sizeof(float)
            : 0;
    return (carries + 255) / 256 * 256;
}

template <typename T, int N, bool HEADS, bool OUTPUT, bool HAS_Z, int CONV, bool DTWS>
void launch_pass(const ScanKParams& p, bool softplus, dim3 grid, hipStream_t stream) {
    if (softplus)
        hipLaunchKernelGGL((scan_chunk_kernel<T, N, HEADS, OUTPUT, HAS_Z, true, CONV, DTWS>), grid, dim3(kScanBlock), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((scan_chunk_kernel<T, N, HEADS, OUTPUT, HAS_Z, false, CONV, DTWS>), grid, dim3(kScanBlock), 0,
                           stream, p);
}

template <typename T, int N, bool HEADS, bool DTWS>
hipError_t launch_scan_typed(const ScanArgs& a, const ScanPlan& plan) {
    ScanKParams p;
    p.u = a.u; p.delta = a.delta; p.A = a.A; p.B = a.B; p.C = a.C; p.D = a.D; p.z = a.z;
    p.delta_bias = a.delta_bias; p.doc_start = a.doc_start; p.initial_state = a.initial_state;
    p.out = a.out; p.final_state = a.final_state;
    const int64_t count = a.batch * a.dim * N;
    const int64_t nslots = plan.nchunks - 1;
    p.ws_P = a.ws;
    p.ws_H = a.ws ? a.ws + nslots * count : nullptr;
    p.dt_ws = (DTWS && a.ws) ? reinterpret_cast<char*>(a.ws) + dt_ws_offset(a.batch, a.dim, N, plan) : nullptr;
    p.seqlen = a.seqlen;
    p.chunk_len = plan.chunk_len;
    p.dim = static_cast<int>(a.dim);
    p.nheads = a.nheads;
    p.headdim = a.nheads ? static_cast<int>(a.dim / a.nheads) : 0;
    p.nbatch = static_cast<int>(a.batch);
    p.softplus = a.softplus ? 1 : 0;
    p.conv_x = a.conv_x; p.conv_w = a.conv_w; p.conv_b = a.conv_b; p.conv_state = a.conv_state;
    p.u_out = a.conv_x ? const_cast<void*>(a.u) : nullptr;
    p.nslots = nslots;

    constexpr int64_t LPC = (HEADS && N > 16) ? N / 16 : 1;     // lanes per channel (as in the kernel)
    const unsigned gx = static_cast<unsigned>((a.dim * LPC + kScanBlock - 1) / kScanBlock);
    const dim3 gall(gx, static_cast<unsigned>(plan.nchunks), static_cast<unsigned>(a.batch));
    // Without a u output the conv is formed in both passes, else pass 3 reads u.
    const bool store_u = p.u_out != nullptr;
    // Pass 1 runs on every chunk when it also produces something the last chunk
    // needs (u of the fused conv, the handed-over step sizes); otherwise on every
    // chunk but the last.
    const bool pass1_all = (a.conv_x != nullptr && store_u) || DTWS;
    if (pass1_all || nslots > 0) {
        const dim3 g1 = pass1_all ? gall : dim3(gx, static_cast<unsigned>(nslots), static_cast<unsigned>(a.batch));
        if constexpr (!HEADS) {
            if (a.conv_x != nullptr && store_u)
                launch_pass<T, N, false, false, false, kConvStoreU, DTWS>(p, a.softplus, g1, a.stream);
            else if (a.conv_x != nullptr)
                launch_pass<T, N, false, false, false, kConvNoStore, DTWS>(p, a.softplus, g1, a.stream);
            else
                launch_pass<T, N, false, false, false, kConvNone, DTWS>(p, a.softplus, g1, a.stream);
        } else {
            launch_pass<T, N, true, false, false, kConvNone, false>(p, a.softplus, g1, a.stream);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (nslots > 0) {
        dim3 g2(static_cast<unsigned>((count + 255) / 256));
        hipLaunchKernelGGL(scan_carry_kernel, g2, dim3(256), 0, a.stream, p.ws_P, p.ws_H, a.initial_state, count,
                           nslots);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int kConv3 = HEADS ? kConvNone : kConvNoStore;
    const bool conv3 = !HEADS && a.conv_x != nullptr && !store_u;
    if (a.z) {
        if (conv3) launch_pass<T, N, HEADS, true, true, kConv3, DTWS>(p, a.softplus, gall, a.stream);
        else launch_pass<T, N, HEADS, true, true, kConvNone, DTWS>(p, a.softplus, gall, a.stream);
    } else {
        if (conv3) launch_pass<T, N, HEADS, true, false, kConv3, DTWS>(p, a.softplus, gall, a.stream);
        else launch_pass<T, N, HEADS, true, false, kConvNone, DTWS>(p, a.softplus, gall, a.stream);
    }
    return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_scan_channels(const ScanArgs& a, const ScanPlan& plan) {
    return a.dt_handoff ? launch_scan_typed<T, N, false, true>(a, plan) : launch_scan_typed<T, N, false, false>(a, plan);
}

template <typename T>
hipError_t launch_scan_dtype(const ScanArgs& a, const ScanPlan& plan) {
    switch (a.dstate) {
        case 4: return launch_scan_channels<T, 4>(a, plan);
        case 8: return launch_scan_channels<T, 8>(a, plan);
        case 16: return launch_scan_channels<T, 16>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

// Scalar-A heads with fp32 I/O keep the recurrent form (fp32 throughout): the
// matrix-core form rounds its operands to bf16, below what fp32 I/O promises.
hipError_t launch_heads_f32(const ScanArgs& a, const ScanPlan& plan) {
    switch (a.dstate) {
        case 16: return launch_scan_typed<float, 16, true, false>(a, plan);
        case 32: return launch_scan_typed<float, 32, true, false>(a, plan);
        case 64: return launch_scan_typed<float, 64, true, false>(a, plan);
        case 128: return launch_scan_typed<float, 128, true, false>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t scan_kernel_dstate(int64_t dim, int64_t dstate, int nheads, bool bf16) {
    if (dstate < 1) return 0;
    if (nheads == 0) return dstate <= 4 ? 4 : dstate <= 8 ? 8 : dstate <= 16 ? 16 : 0;
    if (bf16) {
        const int64_t nt = (dstate + 7) / 8 * 8;
        return ssd_supported(dim, nt, nheads) ? nt : 0;
    }
    for (int64_t nt = 16; nt <= 128; nt *= 2)
        if (dstate <= nt) return nt;
    return 0;
}

bool scan_supported(int64_t dim, int64_t dstate, int nheads, bool bf16) {
    return scan_kernel_dstate(dim, dstate, nheads, bf16) != 0;
}

// Chunks are sized for enough waves per pass: about 8192 (two rounds of four
// waves per SIMD on 256 CUs) while a chunk keeps at least 512 tokens, else about
// 4096.  The chunk is the largest power of two not above the length that gives
// that count: rounding up instead left wide rows (one row of 5120 channels) at
// 2.5 waves per SIMD and 20% slower; 8192 waves with 512-token chunks run a
// 64K-token row of 5120 channels 3.5% faster than 5120 waves with 1024, while
// two 32K rows of 1536 channels are fastest at 6144 waves with 256 (128 and 512
// are 2.5% slower).  Below 128 tokens per chunk the per-chunk overhead wins.
ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim) {
    const int64_t chains = batch * ((dim + 63) / 64);
    auto chunk_for = [&](int64_t target_waves) {
        int64_t want_chunks = chains > 0 ? (target_waves + chains - 1) / chains : 1;
        if (want_chunks < 1) want_chunks = 1;
        const int64_t len = (seqlen + want_chunks - 1) / want_chunks;
        int64_t chunk = 128;
        while (chunk * 2 <= len) chunk *= 2;
        return chunk > 4096 ? int64_t(4096) : chunk;
    };
    int64_t chunk = chunk_for(2 * MAMBA_SCAN_TARGET_WAVES);
    if (chunk < 512) chunk = chunk_for(MAMBA_SCAN_TARGET_WAVES);
    ScanPlan p;
    p.chunk_len = chunk;
    p.nchunks = seqlen > 0 ? (seqlen + chunk - 1) / chunk : 0;
    return p;
}

// fp32 scalar-A heads give each channel dstate / 16 lanes (all of them for
// fewer): the chunk plan counts those lanes as channels.
static int64_t heads_f32_lanes(int64_t dstate) { return dstate > 16 ? dstate / 16 : 1; }

size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads, bool bf16,
                            bool dt_handoff) {
    if (nheads > 0 && bf16) return ssd_workspace_bytes(batch, seqlen, dim, dstate, nheads);
    const ScanPlan plan = plan_scan(batch, seqlen, nheads > 0 ? dim * heads_f32_lanes(dstate) : dim);
    const size_t carries =
        plan.nchunks > 1
            ? static_cast<size_t>(2 * (plan.nchunks - 1)) * static_cast<size_t>(batch * dim * dstate) * sizeof(float)
            : 0;
    if (nheads > 0 || !dt_handoff) return carries;
    // Per-channel A: the step sizes pass 1 hands to pass 3 follow the carries.
    return dt_ws_offset(batch, dim, dstate, plan) +
           static_cast<size_t>(batch * seqlen * dim) * (bf16 ? 2 : 4);
}

hipError_t launch_selective_scan(const ScanArgs& a) {
    if (a.nheads > 0)
        return a.bf16 ? launch_ssd(a)
                      : launch_heads_f32(a, plan_scan(a.batch, a.seqlen, a.dim * heads_f32_lanes(a.dstate)));
    const ScanPlan plan = plan_scan(a.batch, a.seqlen, a.dim);
    return a.bf16 ? launch_scan_dtype<bf16_t>(a, plan) : launch_scan_dtype<float>(a, plan);
}

}  // namespace mamba
