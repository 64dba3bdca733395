// Scalar-A heads (the Mamba-2 shape) as chunked matrix products on the matrix
// cores, gfx950.
//
// Mamba skill page, "Mamba-2: Structured State Space Duality (SSD)": when A is
// one scalar per head the recurrence inside a chunk equals a causal, decay-
// weighted product of C against B (an attention-like Q x Q matrix), and chunks
// talk to each other only through the N x P state of each head.  For one row b,
// one head h (channels h*P .. h*P + P - 1) and a chunk of Q = 64 tokens:
//
//   dt_t    = softplus(delta[t, h] + delta_bias[h])
//   cs_t    = log2(e) A[h] (dt_0 + ... + dt_t)          (inclusive, inside the chunk)
//   seg_t   = number of document starts at or before t  (inside the chunk)
//   M[t, s] = (C_t . B_s) 2^(cs_t - cs_s) dt_s   if s <= t and seg_t == seg_s, else 0
//   Y[t, :] = sum_s M[t, s] x_s  +  [seg_t == 0] 2^cs_t  C_t . H_in
//   H_out   = [seg_63 == 0] 2^cs_63 H_in  +  sum_s [seg_s == seg_63] 2^(cs_63 - cs_s) dt_s B_s x_s^T
//   out_t   = (Y[t, :] + D x_t) * silu(z_t)
//
// This is the same recurrence as h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t with
// the state zeroed at every document start, regrouped (exactly, up to rounding).
// Every product runs as v_mfma_f32_16x16x32_bf16: bf16 operands (inputs are
// bf16 already; M, dt-weighted B and the chunk-entry state are rounded to bf16)
// and fp32 accumulation.  The state H of a head lives in fp32 MFMA accumulators
// across all chunks of a segment.
//
// Parallelism: one workgroup (8 waves) per (row, head, segment of L).
// Segments are joined like the chunks of the per-channel scan: pass 1 computes
// every segment's end state from zero and its total decay, pass 2 carries the
// states across segments, pass 3 recomputes each segment from its carry and
// writes the outputs.  Workgroups of the same (row, segment) read the same B and
// C rows, so the block index is remapped to keep all heads of one (row, segment)
// on one XCD (the dispatcher deals consecutive workgroups round-robin to the 8
// XCDs, each with its own L2).
//
// Work of wave w in a chunk: half of output row tile w / 2 (tokens 16 (w / 2) ..
// + 15, channel half w % 2), half of the C B^T tiles of that row, and state
// tiles k = w, w + 8, ...  Its C rows come straight from global memory into MFMA
// fragments; B, x and the per-token scalars are shared through LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace mamba {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;                  // tokens per chunk
#ifndef MAMBA_SSD_WAVES
#define MAMBA_SSD_WAVES 8               // waves per workgroup: 8, or 4 (two workgroups per CU)
#endif
constexpr int kWaves = MAMBA_SSD_WAVES;
static_assert(kWaves == 4 || kWaves == 8, "one or two waves per 16-token output row tile");
constexpr int kRowW = kWaves / 4;       // waves sharing one 16-token output row tile
constexpr int kThreads = 64 * kWaves;
// B rows, x^T and the per-token scalars double-buffered by chunk parity (no
// barrier between chunks), or single-buffered (a barrier at each chunk's end,
// and an LDS footprint that lets two 4-wave workgroups share a CU).
#ifndef MAMBA_SSD_DBUF
#define MAMBA_SSD_DBUF (MAMBA_SSD_WAVES == 8)
#endif
constexpr int kBuf = MAMBA_SSD_DBUF ? 2 : 1;
#ifndef MAMBA_SSD_TARGET_BLOCKS
#define MAMBA_SSD_TARGET_BLOCKS 768
#endif
constexpr int64_t kTargetBlocks = MAMBA_SSD_TARGET_BLOCKS;  // workgroups per pass
constexpr int kXcds = 8;
// The fused conv (template argument CONV): used when the caller wants no u.  With
// u wanted, the conv kernel writes it first: forming u in the aggregate pass
// costs that latency-bound pass more than the conv kernel's own pass over x and
// u (549 against 520 us per call on 2 x 32768 tokens, 24 heads, N = 128).
constexpr int kConvNone = 0;            // the activations loaded are u
constexpr int kConvForm = 1;            // loaded x; u formed (not stored)
#ifndef MAMBA_SSD_WAVES_PER_EU
#define MAMBA_SSD_WAVES_PER_EU 2        // up to 256 VGPRs: one 8-wave workgroup per CU
#endif

struct SsdParams {
    const uint16_t* u;
    const uint16_t* delta;
    const float* A;
    const uint16_t* B;
    const uint16_t* C;
    const float* D;
    const uint16_t* z;
    const float* delta_bias;
    const uint8_t* doc_start;
    const float* initial_state;   // (B, D, N) or null: state before token 0
    uint16_t* out;
    float* final_state;
    const uint16_t* conv_x;       // fused conv: its input x (B, L, D), or null (u is given)
    const float* conv_w;          // (D, 4)
    const float* conv_b;          // (D,) or null
    const uint16_t* conv_state;   // (B, D, 3) or null: x of the three tokens before token 0
    float* ws_H;        // [B*H][nseg-1][P][N]: segment end states, then carries
    float* ws_G;        // [B*H][nseg-1]: segment decays
    int64_t seqlen;
    int64_t seg_len;    // multiple of kQ
    int dim;
    int nheads;
    int dstate;
    int nseg;
    int nbatch;
};

__device__ __forceinline__ bf16x8_t frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// D = A x B + C for a 16x16 tile, K = 32.  Lane l holds A[l % 16][8 (l / 16) + j]
// and B[8 (l / 16) + j][l % 16] (j = 0..7); D[4 (l / 16) + i][l % 16] (i = 0..3).
__device__ __forceinline__ f32x4_t mma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }


// Makes v a value defined here, so later uses do not wait on the load it came
// from (a wait there would also drain every load issued after it).
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(u32x4_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    constexpr int kRsrcWord3 = 0x00020000;        // gfx9 data format: 32-bit, raw access
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Row padding of the LDS tiles, in elements (tunable; fragment loads need the
// bf16 row strides to stay multiples of 8 elements, the fp32 one of 4).
#ifndef MAMBA_SSD_PAD_N
#define MAMBA_SSD_PAD_N 8
#endif
#ifndef MAMBA_SSD_PAD_Q
#define MAMBA_SSD_PAD_Q 16
#endif
#ifndef MAMBA_SSD_PAD_Y
#define MAMBA_SSD_PAD_Y 4
#endif

// LDS layout of one workgroup.  Row strides carry padding so that the 16 rows
// read by one fragment load start on different banks: 8 bf16 for the [*][N]
// tiles; 16 bf16 for the [*][Q] tiles, whose transposing 2-byte stores (x^T, M,
// dt-weighted B^T) conflict least at that stride (measured on the 32K heads
// shape: 518 us per call against 535 with 8, 553-569 with 24-56).
template <int NP, int P, bool OUTPUT>
struct SsdLds {
    static constexpr int SN = NP + MAMBA_SSD_PAD_N;        // [*][NP] bf16 tiles
    static constexpr int SQ = kQ + MAMBA_SSD_PAD_Q;        // [*][Q] bf16 tiles
    static constexpr int SY = P / kRowW + MAMBA_SSD_PAD_Y; // per-wave fp32 output tile [16][SY]
    static_assert(SN % 8 == 0 && SQ % 8 == 0 && SY % 4 == 0, "row strides of the fragment and vector accesses");
    static constexpr int kBBytes = kQ * SN * 2;
    static constexpr int kYBytes = OUTPUT ? kWaves * 16 * SY * 4 : 0;
    // B rows, x^T and the per-token scalars: kBuf copies (chunk parity).
    static constexpr int kBRegion = kBBytes > kYBytes ? kBBytes : kYBytes;
    static constexpr int oB = 0;                                    // kBuf x B rows [s][n]; later the output tiles
    static constexpr int oBw = oB + kBuf * kBRegion;                // dt-weighted B^T [n][s]
    static constexpr int oXT = oBw + NP * SQ * 2;                   // kBuf x x^T [p][s]
    static constexpr int oM = oXT + kBuf * P * SQ * 2;              // M [t][s]
    static constexpr int oHT = oM + (OUTPUT ? kQ * SQ * 2 : 0);     // chunk-entry state^T [p][n]
    static constexpr int oTok = oHT + (OUTPUT ? P * SN * 2 : 0);    // kBuf x per-token scalars
    static constexpr int oCw = oTok + kBuf * 5 * kQ * 4;            // fused conv: taps [P][4], bias [P]
    static constexpr int kBytes = oCw + P * 5 * 4;
};

template <int NP, int P, bool OUTPUT, bool HAS_Z, bool SOFTPLUS, int CONV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MAMBA_SSD_WAVES_PER_EU))) void ssd_chunk_kernel(
    const SsdParams p) {
    using Lay = SsdLds<NP, P, OUTPUT>;
    constexpr int SN = Lay::SN, SQ = Lay::SQ, SY = Lay::SY;
    constexpr int kTN = NP / 16, kTP = P / 16;
    constexpr int kT = kTN * kTP;                          // state tiles
    constexpr int kSt = (kT + kWaves - 1) / kWaves;        // state tiles per wave
    constexpr int kKB = NP / 32;                           // K blocks over the states
    constexpr int kVN = NP / 8;                            // 16-byte vectors per B row
    constexpr int kBV = (kQ * kVN + kThreads - 1) / kThreads;
    constexpr int kPW = P / kRowW;                         // channels of a wave's output tile part
    constexpr int kTPW = kPW / 16;                         // its 16-channel tiles
    constexpr int kLPR = kPW / 8;                          // lanes per token row (8 channels each)
    constexpr int kBwTasks = (kQ / 2) * kVN;               // (token pair, 8 states) tasks

    __shared__ __attribute__((aligned(16))) unsigned char lds[Lay::kBytes];
    uint16_t* sB0 = reinterpret_cast<uint16_t*>(lds + Lay::oB);
    uint16_t* sBw = reinterpret_cast<uint16_t*>(lds + Lay::oBw);
    uint16_t* sXT0 = reinterpret_cast<uint16_t*>(lds + Lay::oXT);
    uint16_t* sM = reinterpret_cast<uint16_t*>(lds + Lay::oM);
    uint16_t* sHT = reinterpret_cast<uint16_t*>(lds + Lay::oHT);
    float* sTok0 = reinterpret_cast<float*>(lds + Lay::oTok);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;


    // Workgroup -> (row, segment, head); all heads of a (row, segment) share an XCD.
    const int total = p.nbatch * p.nheads * p.nseg;
    int li = static_cast<int>(blockIdx.x);
    if (total % kXcds == 0) li = (li % kXcds) * (total / kXcds) + li / kXcds;
    const int h = li % p.nheads;
    const int bs = li / p.nheads;
    const int seg = bs % p.nseg;
    const int b = bs / p.nseg;
    if (!OUTPUT && seg == p.nseg - 1) return;      // the last segment's aggregate is never used

    const int64_t L = p.seqlen;
    const int N = p.dstate;
    const int64_t t_seg0 = static_cast<int64_t>(seg) * p.seg_len;
    const int64_t t_seg1 = (t_seg0 + p.seg_len < L) ? t_seg0 + p.seg_len : L;
    const float a_l2 = p.A[h] * kLog2e;
    const float dbias = p.delta_bias ? p.delta_bias[h] : 0.0f;
    const int64_t bh = static_cast<int64_t>(b) * p.nheads + h;
    const int64_t PN = static_cast<int64_t>(P) * N;
    const int nslot = p.nseg - 1;
    const uint16_t* Brow = p.B + static_cast<int64_t>(b) * L * N;
    const uint16_t* Crow = p.C + static_cast<int64_t>(b) * L * N;

    // State tiles of this wave: tile k = wave + kWaves j covers n in 16 (k / kTP) + [0, 16)
    // and p in 16 (k % kTP) + [0, 16); lane element i is (n = 16 nb + 4 lg + i, p = 16 pb + l16).
    f32x4_t st[kSt];
#pragma unroll
    for (int j = 0; j < kSt; ++j) {
        const int k = wave + kWaves * j;
        st[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (OUTPUT && (seg > 0 || p.initial_state != nullptr) && k < kT) {
            const int nb = k / kTP, pb = k % kTP;
            const float* carry = (seg > 0 ? p.ws_H + (bh * nslot + seg - 1) * PN : p.initial_state + bh * PN) +
                                 static_cast<int64_t>(16 * pb + l16) * N;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 16 * nb + 4 * lg + i;
                if (n < N) st[j][i] = carry[n];
            }
        }
    }
    float seg_decay = 1.0f;

    // This wave's part of the chunk: output row tile `wt` (tokens 16 wt ..), channels
    // wp .. wp + kPW - 1.  x staging and the epilogue: lane -> tokens x_row + kXStep r
    // (r < kXR), channels x_p0 .. x_p0 + 7 (lanes past kXL idle).
    constexpr int kXL = 16 * kLPR < 64 ? 16 * kLPR : 64;   // lanes that stage x rows
    constexpr int kXR = 16 * kLPR / kXL;                    // x rows per lane
    constexpr int kXStep = 64 / kLPR;                       // token step between a lane's rows
    const int wt = wave / kRowW;
    const int wp = (wave % kRowW) * kPW;
    const bool x_lane = lane < kXL;
    const int x_row = 16 * wt + (x_lane ? lane / kLPR : 0);
    const int x_p0 = wp + (lane % kLPR) * 8;
    float Dp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) Dp[e] = (OUTPUT && p.D) ? p.D[h * P + x_p0 + e] : 0.0f;
    // Fused conv: the taps and bias of the head's channels, in LDS (read per chunk:
    // 40 registers per lane would halve the aggregate pass's occupancy).
    float* sCw = reinterpret_cast<float*>(lds + Lay::oCw);
    float* sCb = sCw + 4 * P;
    if constexpr (CONV != kConvNone) {
        if (tid < 4 * P) sCw[tid] = p.conv_w[static_cast<int64_t>(h) * P * 4 + tid];
        if (tid < P) sCb[tid] = p.conv_b ? p.conv_b[h * P + tid] : 0.0f;
        lds_barrier();
    }

    // Global data of one chunk, held in registers one chunk ahead so that its
    // loads overlap the current chunk's work.  Every load is unconditional (token
    // and state indices clamped into range): rows past the segment end only ever
    // meet a zero step size, and padded states are zeroed when consumed.
    u32x4_t pb_[kBV], pc_[kKB], px_[kXR], pz_[kXR];
    uint32_t pdelta = 0, pflag = 0;
    // Fused conv: x of the three tokens before each of this lane's tokens (row
    // offsets 1..3) and doc_start of the token and the two before it.
    constexpr int kCH = CONV != kConvNone ? 3 : 1;
    u32x4_t ph_[kXR][kCH];
    uint32_t pf_[kXR][kCH];
    // Buffer resources per row: wave-uniform base and size in SGPRs, 32-bit byte
    // offsets per lane (a row of any tensor is below 2 GiB, checked on the host).
    // A load past a resource's end returns zeros.
    const int64_t arow = L * p.dim;
    const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Brow, L * N * 2);
    const __amdgpu_buffer_rsrc_t rsC = make_rsrc(Crow, L * N * 2);
    const __amdgpu_buffer_rsrc_t rsU = make_rsrc((CONV != kConvNone ? p.conv_x : p.u) + b * arow, arow * 2);
    const __amdgpu_buffer_rsrc_t rsZ = make_rsrc(HAS_Z ? p.z + b * arow : nullptr, HAS_Z ? arow * 2 : 0);
    const __amdgpu_buffer_rsrc_t rsDl = make_rsrc(p.delta + b * L * p.nheads, L * p.nheads * 2);
    const __amdgpu_buffer_rsrc_t rsDs = make_rsrc(p.doc_start ? p.doc_start + b * L : nullptr, p.doc_start ? L : 0);
    const int xcol = h * P + x_p0;
    auto fetch = [&](int64_t c0) {
        const int c0i = static_cast<int>(c0);
#pragma unroll
        for (int k = 0; k < kBV; ++k) {
            const int i = tid + kThreads * k;
            if (i < kQ * kVN) {
                const int row = i / kVN, n0 = (i % kVN) * 8;
                pb_[k] = load16(rsB, ((c0i + row) * N + n0) * 2);
            }
        }
        if constexpr (OUTPUT) {
            const int cbase = ((c0i + 16 * wt + l16) * N + 8 * lg) * 2;
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) pc_[kb] = load16(rsC, cbase + 64 * kb);
        }
#pragma unroll
        for (int r = 0; r < kXR; ++r) {
            const int xr = x_row + kXStep * r;
            const int xoff = ((c0i + xr) * p.dim + xcol) * 2;
            px_[r] = load16(rsU, xoff);
            if constexpr (CONV != kConvNone) {
                // Rows before the row start give negative offsets: past the resource
                // (as unsigned), so they load zeros, as do flags past the row.
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    ph_[r][k] = load16(rsU, xoff - (k + 1) * p.dim * 2);
                    pf_[r][k] = __builtin_amdgcn_raw_buffer_load_b8(rsDs, c0i + xr - k, 0, 0);
                }
            }
            if (OUTPUT && HAS_Z) pz_[r] = load16(rsZ, xoff);
        }
        if (wave == 0) {
            pdelta = __builtin_amdgcn_raw_buffer_load_b16(rsDl, ((c0i + lane) * p.nheads + h) * 2, 0, 0);
            pflag = __builtin_amdgcn_raw_buffer_load_b8(rsDs, c0i + lane, 0, 0);
        }
    };

    // Let the loads above (carry, D) land before the chunk loop: otherwise the wait
    // for them sits inside the loop and also drains every chunk's prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    if (t_seg0 < t_seg1) fetch(t_seg0);
    const u32x4_t kZero = {0u, 0u, 0u, 0u};
    for (int64_t t0 = t_seg0; t0 < t_seg1; t0 += kQ) {
        const int par = kBuf == 2 ? static_cast<int>(((t0 - t_seg0) / kQ) & 1) : 0;
        uint16_t* sB = sB0 + par * (Lay::kBRegion / 2);
        uint16_t* sXT = sXT0 + par * P * SQ;
        float* sDt = sTok0 + par * 5 * kQ;
        float* sCs = sDt + kQ;
        float* sW = sCs + kQ;
        float* sScale = sW + kQ;
        int* sSeg = reinterpret_cast<int*>(sScale + kQ);
        float* sYw = reinterpret_cast<float*>(sB) + wave * 16 * SY;   // this wave's output tile (over B rows)
        // ---- 1. take the prefetched chunk: u (formed by the fused conv), B rows to
        //         LDS, u transposed to LDS, per-token scalars, this wave's C
        //         fragments, the gate
        u32x4_t cx[kXR], cz[kXR];
#pragma unroll
        for (int r = 0; r < kXR; ++r) {
            cx[r] = px_[r];
            cz[r] = kZero;
            pin(cx[r]);
        }
        if constexpr (CONV != kConvNone) {
#pragma unroll
            for (int r = 0; r < kXR; ++r) {
                const int xr = x_row + kXStep * r;
                u32x4_t hx[3];
                uint32_t fl[3];
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    hx[k] = ph_[r][k];
                    fl[k] = pf_[r][k];
                    pin(hx[k]);
                    pin(fl[k]);
                }
                if (p.conv_state != nullptr && t0 + xr < 3) {
                    // the given history before token 0: (B, D, 3), oldest first
                    const uint16_t* cs = p.conv_state + (static_cast<int64_t>(b) * p.dim + h * P + x_p0) * 3;
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        const int rr = static_cast<int>(t0) + xr - (k + 1);
                        if (rr < 0) {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                hx[k][j] = static_cast<uint32_t>(cs[(2 * j) * 3 + 3 + rr]) |
                                           (static_cast<uint32_t>(cs[(2 * j + 1) * 3 + 3 + rr]) << 16);
                        }
                    }
                }
                // A document start at the token (or one or two before it) cuts the
                // taps that reach past it: they read zero, as in the conv kernel.
                const bool c1 = fl[0] == 0, c2 = c1 && fl[1] == 0, c3 = c2 && fl[2] == 0;
                const float4 cb0 = *reinterpret_cast<const float4*>(sCb + x_p0);
                const float4 cb1 = *reinterpret_cast<const float4*>(sCb + x_p0 + 4);
                const float cbias[8] = {cb0.x, cb0.y, cb0.z, cb0.w, cb1.x, cb1.y, cb1.z, cb1.w};
                uint32_t uo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float uv[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int e = 2 * j + q;
                        const float4 w = *reinterpret_cast<const float4*>(sCw + (x_p0 + e) * 4);
                        auto el = [&](uint32_t v) { return q == 0 ? lo_bf16(v) : hi_bf16(v); };
                        const float h1 = c1 ? el(hx[0][j]) : 0.0f;
                        const float h2 = c2 ? el(hx[1][j]) : 0.0f;
                        const float h3 = c3 ? el(hx[2][j]) : 0.0f;
                        float acc = __builtin_fmaf(w.w, el(cx[r][j]), cbias[e]);
                        acc = __builtin_fmaf(w.z, h1, acc);
                        acc = __builtin_fmaf(w.y, h2, acc);
                        acc = __builtin_fmaf(w.x, h3, acc);
                        uv[q] = silu_f(acc);
                    }
                    uo[j] = pack2(uv[0], uv[1]);
                }
                cx[r] = u32x4_t{uo[0], uo[1], uo[2], uo[3]};
            }
        }
#pragma unroll
        for (int k = 0; k < kBV; ++k) {
            const int i = tid + kThreads * k;
            if (i < kQ * kVN) {
                const int row = i / kVN, n0 = (i % kVN) * 8;
                *reinterpret_cast<u32x4_t*>(sB + row * SN + n0) = (n0 < N) ? pb_[k] : kZero;
            }
        }
        u32x4_t cf[kKB];
        if constexpr (OUTPUT) {
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                cf[kb] = (32 * kb + 8 * lg < N) ? pc_[kb] : kZero;
                pin(cf[kb]);
            }
        }
        if constexpr (OUTPUT && HAS_Z) {
#pragma unroll
            for (int r = 0; r < kXR; ++r) {
                cz[r] = pz_[r];
                pin(cz[r]);
            }
        }
        if (x_lane) {
#pragma unroll
            for (int r = 0; r < kXR; ++r) {
                const int xr = x_row + kXStep * r;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sXT[(x_p0 + 2 * j) * SQ + xr] = static_cast<uint16_t>(cx[r][j] & 0xffffu);
                    sXT[(x_p0 + 2 * j + 1) * SQ + xr] = static_cast<uint16_t>(cx[r][j] >> 16);
                }
            }
        }
        if (wave == 0) {
            // Lane = token of the chunk.  Tokens past the segment end are identity
            // steps (dt = 0).
            const int64_t tg = t0 + lane;
            const bool valid = tg < t_seg1;
            float dt = 0.0f;
            if (valid) {
                dt = bf16_to_f32(static_cast<uint16_t>(pdelta)) + dbias;
                if constexpr (SOFTPLUS) dt = softplus_f(dt);
            }
            // Token 0 starts a document unless the row continues an initial state.
            const bool reset = valid && ((tg == 0 && p.initial_state == nullptr) || pflag != 0);
            const float cs = wave_prefix_sum(dt * a_l2);
            const uint64_t rmask = __ballot(reset);
            const int sg = __popcll(rmask & ((2ull << lane) - 1ull));
            const int sg_end = __popcll(rmask);
            const float cs_end = lane_value(cs, 63);
            sDt[lane] = dt;
            sCs[lane] = cs;
            sSeg[lane] = sg;
            sW[lane] = (sg == sg_end) ? exp2_fast(cs_end - cs) * dt : 0.0f;
            sScale[lane] = (sg == 0) ? exp2_fast(cs) : 0.0f;
        }
        if (t0 + kQ < t_seg1) fetch(t0 + kQ);
        lds_barrier();

        // ---- 2. M = mask(C B^T): this wave's share of row tile wt; the chunk-entry
        //         state as bf16; dt-weighted B^T
        if constexpr (OUTPUT) {
            const int ti = wt;
            const int kread = 2 * (ti / 2 + 1);            // column tiles of M read by row tile ti
            float cs_t[4];
            int sg_t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs_t[i] = sCs[16 * ti + 4 * lg + i];
                sg_t[i] = sSeg[16 * ti + 4 * lg + i];
            }
#pragma unroll
            for (int tj = wave % kRowW; tj < 4; tj += kRowW) {
                if (tj >= kread) break;
                f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
                if (tj <= ti) {
#pragma unroll
                    for (int kb = 0; kb < kKB; ++kb)
                        g = mma(__builtin_bit_cast(bf16x8_t, cf[kb]),
                                frag(sB + (16 * tj + l16) * SN + 32 * kb + 8 * lg), g);
                }
                const int s = 16 * tj + l16;
                const float cs_s = sCs[s], dt_s = sDt[s];
                const int sg_s = sSeg[s];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * ti + 4 * lg + i;
                    // Computed for every element, then selected: for s > t the
                    // exponent can be positive, and the select drops any inf.
                    const float m = g[i] * exp2_fast(cs_t[i] - cs_s) * dt_s;
                    sM[t * SQ + s] = f32_to_bf16((s <= t && sg_t[i] == sg_s) ? m : 0.0f);
                }
            }
#pragma unroll
            for (int j = 0; j < kSt; ++j) {
                const int k = wave + kWaves * j;
                if (k < kT) {
                    const int nb = k / kTP, pb = k % kTP;
                    const u32x2_t v = {pack2(st[j][0], st[j][1]), pack2(st[j][2], st[j][3])};
                    *reinterpret_cast<u32x2_t*>(sHT + (16 * pb + l16) * SN + 16 * nb + 4 * lg) = v;
                }
            }
        }
        // dt-weighted B^T, two tokens per task so each write is one 32-bit word;
        // token pairs run along the lanes, so the writes hit consecutive words.
        for (int i = tid; i < kBwTasks; i += kThreads) {
            const int s = 2 * (i % (kQ / 2)), n0 = (i / (kQ / 2)) * 8;
            const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(sB + s * SN + n0);
            const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(sB + (s + 1) * SN + n0);
            const float w0 = sW[s], w1 = sW[s + 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *reinterpret_cast<uint32_t*>(sBw + (n0 + 2 * j) * SQ + s) =
                    pack2(lo_bf16(v0[j]) * w0, lo_bf16(v1[j]) * w1);
                *reinterpret_cast<uint32_t*>(sBw + (n0 + 2 * j + 1) * SQ + s) =
                    pack2(hi_bf16(v0[j]) * w0, hi_bf16(v1[j]) * w1);
            }
        }
        lds_barrier();

        // ---- 3. products: Y = scale (C H_in) + M x for this wave's output tiles;
        //         H = g H + (dt-weighted B)^T x for its state tiles
        const float g_chunk = sScale[kQ - 1];
        f32x4_t y[kTPW];
        if constexpr (OUTPUT) {
            const int ti = wt;
            float scale[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) scale[i] = sScale[16 * ti + 4 * lg + i];
#pragma unroll
            for (int tp = 0; tp < kTPW; ++tp) {
                y[tp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
                    y[tp] = mma(__builtin_bit_cast(bf16x8_t, cf[kb]),
                                frag(sHT + (wp + 16 * tp + l16) * SN + 32 * kb + 8 * lg), y[tp]);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[tp][i] *= scale[i];
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb > ti / 2) break;
                const bf16x8_t a = frag(sM + (16 * ti + l16) * SQ + 32 * kb + 8 * lg);
#pragma unroll
                for (int tp = 0; tp < kTPW; ++tp)
                    y[tp] = mma(a, frag(sXT + (wp + 16 * tp + l16) * SQ + 32 * kb + 8 * lg), y[tp]);
            }
        }
#pragma unroll
        for (int j = 0; j < kSt; ++j) {
            const int k = wave + kWaves * j;
            if (k < kT) {
                const int nb = k / kTP, pb = k % kTP;
                st[j] *= g_chunk;
#pragma unroll
                for (int kb = 0; kb < kQ / 32; ++kb)
                    st[j] = mma(frag(sBw + (16 * nb + l16) * SQ + 32 * kb + 8 * lg),
                                frag(sXT + (16 * pb + l16) * SQ + 32 * kb + 8 * lg), st[j]);
            }
        }
        seg_decay *= g_chunk;

        // ---- 4. outputs of this wave's tiles: they go through the wave's own LDS
        //         area (over the B rows, which every wave is done with) to a
        //         token-per-lane layout, then (Y + D x) silu(z) as bf16 rows
        if constexpr (OUTPUT) {
#pragma unroll
            for (int tp = 0; tp < kTPW; ++tp)
#pragma unroll
                for (int i = 0; i < 4; ++i) sYw[(4 * lg + i) * SY + 16 * tp + l16] = y[tp][i];
#pragma unroll
            for (int r = 0; r < kXR; ++r) {
                const int xr = x_row + kXStep * r;
                const int64_t tx = t0 + xr;
                if (x_lane && tx < t_seg1) {
                    const float* yr = sYw + (xr - 16 * wt) * SY + (x_p0 - wp);
                    uint32_t o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float y0 = __builtin_fmaf(Dp[2 * j], lo_bf16(cx[r][j]), yr[2 * j]);
                        float y1 = __builtin_fmaf(Dp[2 * j + 1], hi_bf16(cx[r][j]), yr[2 * j + 1]);
                        if constexpr (HAS_Z) {
                            y0 *= silu_f(lo_bf16(cz[r][j]));
                            y1 *= silu_f(hi_bf16(cz[r][j]));
                        }
                        o[j] = pack2(y0, y1);
                    }
                    const int64_t off = (static_cast<int64_t>(b) * L + tx) * p.dim + h * P + x_p0;
                    *reinterpret_cast<u32x4_t*>(p.out + off) = u32x4_t{o[0], o[1], o[2], o[3]};
                }
            }
        }
        // Single-buffered: every wave is done with this chunk's B rows (and the
        // output tiles over them), x^T and scalars before the next chunk is staged.
        if constexpr (kBuf == 1) lds_barrier();
    }

#pragma unroll
    for (int j = 0; j < kSt; ++j) {
        const int k = wave + kWaves * j;
        if (k >= kT) continue;
        const int nb = k / kTP, pb = k % kTP;
        const int pp = 16 * pb + l16;
        float* dst;
        if constexpr (OUTPUT) {
            if (seg != p.nseg - 1 || p.final_state == nullptr) continue;
            dst = p.final_state + (static_cast<int64_t>(b) * p.dim + h * P + pp) * N;
        } else {
            dst = p.ws_H + (bh * nslot + seg) * PN + static_cast<int64_t>(pp) * N;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 16 * nb + 4 * lg + i;
            if (n < N) dst[n] = st[j][i];
        }
    }
    if (!OUTPUT && tid == 0) p.ws_G[bh * nslot + seg] = seg_decay;
}

// Pass 2: carry_{k+1} = G_k carry_k + H_k over the segments of each (row, head),
// written over H_k (which then holds the state entering segment k + 1); carry_0
// is the initial state (or zero).  The (B, D, N) initial state of head h of row b
// is the contiguous block (b H + h) P N .. + P N, laid out like H_k.
__global__ __launch_bounds__(256) void ssd_carry_kernel(float* __restrict__ ws_H, const float* __restrict__ ws_G,
                                                        const float* __restrict__ init, int64_t nbh, int nslot,
                                                        int64_t PN) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= nbh * PN) return;
    const int64_t bh = i / PN, e = i % PN;
    float c = init != nullptr ? init[i] : 0.0f;
    for (int k = 0; k < nslot; ++k) {
        float* hp = ws_H + (bh * nslot + k) * PN + e;
        c = __builtin_fmaf(ws_G[bh * nslot + k], c, *hp);
        *hp = c;
    }
}

struct SsdPlan {
    int nseg;
    int64_t seg_len;
};

SsdPlan plan_ssd(int64_t batch, int64_t seqlen, int nheads) {
    SsdPlan s{1, kQ};
    if (seqlen <= 0) return s;
    const int64_t bh = batch * nheads;
    const int64_t nchunks = (seqlen + kQ - 1) / kQ;
    int64_t want = bh > 0 ? (kTargetBlocks + bh - 1) / bh : 1;
    if (want > nchunks) want = nchunks;
    if (want < 1) want = 1;
    const int64_t per_seg = (nchunks + want - 1) / want;
    s.seg_len = per_seg * kQ;
    s.nseg = static_cast<int>((seqlen + s.seg_len - 1) / s.seg_len);
    return s;
}

template <int NP, int P, bool OUTPUT, bool HAS_Z, int CONV>
void launch_chunk(const SsdParams& p, bool softplus, unsigned blocks, hipStream_t stream) {
    if (softplus)
        hipLaunchKernelGGL((ssd_chunk_kernel<NP, P, OUTPUT, HAS_Z, true, CONV>), dim3(blocks), dim3(kThreads), 0, stream,
                           p);
    else
        hipLaunchKernelGGL((ssd_chunk_kernel<NP, P, OUTPUT, HAS_Z, false, CONV>), dim3(blocks), dim3(kThreads), 0,
                           stream, p);
}

template <int NP, int P>
hipError_t launch_ssd_typed(const ScanArgs& a, const SsdPlan& plan) {
    SsdParams p;
    p.u = static_cast<const uint16_t*>(a.u);
    p.delta = static_cast<const uint16_t*>(a.delta);
    p.A = a.A;
    p.B = static_cast<const uint16_t*>(a.B);
    p.C = static_cast<const uint16_t*>(a.C);
    p.D = a.D;
    p.z = static_cast<const uint16_t*>(a.z);
    p.delta_bias = a.delta_bias;
    p.doc_start = a.doc_start;
    p.initial_state = a.initial_state;
    p.out = static_cast<uint16_t*>(a.out);
    p.final_state = a.final_state;
    const int64_t nbh = a.batch * a.nheads;
    const int nslot = plan.nseg - 1;
    const int64_t PN = static_cast<int64_t>(P) * a.dstate;
    p.ws_H = a.ws;
    p.ws_G = a.ws ? a.ws + nbh * nslot * PN : nullptr;
    p.seqlen = a.seqlen;
    p.seg_len = plan.seg_len;
    p.dim = static_cast<int>(a.dim);
    p.nheads = a.nheads;
    p.dstate = static_cast<int>(a.dstate);
    p.nseg = plan.nseg;
    p.nbatch = static_cast<int>(a.batch);
    // Fused conv (no u output): both passes form u from x.
    const bool conv = a.conv_x != nullptr;
    p.conv_x = static_cast<const uint16_t*>(a.conv_x);
    p.conv_w = a.conv_w;
    p.conv_b = a.conv_b;
    p.conv_state = static_cast<const uint16_t*>(a.conv_state);

    const unsigned blocks = static_cast<unsigned>(nbh * plan.nseg);
    if (nslot > 0) {
        if (conv) launch_chunk<NP, P, false, false, kConvForm>(p, a.softplus, blocks, a.stream);
        else launch_chunk<NP, P, false, false, kConvNone>(p, a.softplus, blocks, a.stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t count = nbh * PN;
        hipLaunchKernelGGL(ssd_carry_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0,
                           a.stream, p.ws_H, p.ws_G, a.initial_state, nbh, nslot, PN);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.z) {
        if (conv) launch_chunk<NP, P, true, true, kConvForm>(p, a.softplus, blocks, a.stream);
        else launch_chunk<NP, P, true, true, kConvNone>(p, a.softplus, blocks, a.stream);
    } else {
        if (conv) launch_chunk<NP, P, true, false, kConvForm>(p, a.softplus, blocks, a.stream);
        else launch_chunk<NP, P, true, false, kConvNone>(p, a.softplus, blocks, a.stream);
    }
    return hipGetLastError();
}

template <int NP>
hipError_t launch_ssd_np(const ScanArgs& a, const SsdPlan& plan) {
    switch (a.dim / a.nheads) {
        case 32: return launch_ssd_typed<NP, 32>(a, plan);
        case 64: return launch_ssd_typed<NP, 64>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool ssd_supported(int64_t dim, int64_t dstate, int nheads) {
    if (nheads <= 0 || dim % nheads != 0) return false;
    const int64_t P = dim / nheads;
    return (P == 32 || P == 64) && dstate % 8 == 0 && dstate >= 8 && dstate <= 128;
}

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads) {
    const SsdPlan plan = plan_ssd(batch, seqlen, nheads);
    if (plan.nseg <= 1) return 0;
    const int64_t nbh = batch * nheads;
    const int64_t slots = nbh * (plan.nseg - 1);
    return static_cast<size_t>(slots * (dim / nheads) * dstate + slots) * sizeof(float);
}

hipError_t launch_ssd(const ScanArgs& a) {
    const SsdPlan plan = plan_ssd(a.batch, a.seqlen, a.nheads);
    if (a.dstate <= 32) return launch_ssd_np<32>(a, plan);
    if (a.dstate <= 64) return launch_ssd_np<64>(a, plan);
    return launch_ssd_np<128>(a, plan);
}

}  // namespace mamba
