// Host-side launch descriptors shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mamba {

struct ConvArgs {
    const void* x;
    const float* weight;
    const float* bias;
    const uint8_t* doc_start;
    const void* conv_state;   // (B, D, 3) history before token 0, or null
    void* out;
    int64_t batch, seqlen, dim;
    bool bf16;
    bool vectorized;   // 16-byte loads: dim and pointers aligned
    bool apply_silu;
    hipStream_t stream;
};

hipError_t launch_causal_conv1d(const ConvArgs& a);

// Backward of the conv (conv1d_bwd.hip): dx, dweight, dbias from du.
struct ConvBwdArgs {
    const void* x;
    const float* weight;
    const float* bias;        // or null
    const uint8_t* doc_start;
    const void* du;
    void* dx;
    float* dweight;           // (D, 4)
    float* dbias;             // (D,) or null
    const void* conv_state = nullptr;   // (B, D, 3) inputs before token 0, or null
    float* d_conv_state = nullptr;      // (B, D, 3), written; needs conv_state
    float* ws;                // conv_bwd_workspace_bytes
    int64_t batch, seqlen, dim;
    bool bf16;
    bool vectorized;          // channel pairs: even dim, pointers aligned to two elements
    bool apply_silu;
    hipStream_t stream;
};

size_t conv_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim);
hipError_t launch_causal_conv1d_bwd(const ConvBwdArgs& a);

struct ScanArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* delta_bias;
    const uint8_t* doc_start;
    const float* initial_state;   // (B, D, N) or null
    void* out;
    float* final_state;
    float* ws;          // chunk carries, see scan_workspace_bytes
    // Fused conv1d (width 4, SiLU): when conv_x is set, u is an output: the scan
    // computes u = SiLU(conv(conv_x)) itself (per-channel A) and stores it there.
    const void* conv_x = nullptr;
    const float* conv_w = nullptr;
    const float* conv_b = nullptr;
    const void* conv_state = nullptr;   // (B, D, 3) history before token 0, or null
    int64_t batch, seqlen, dim, dstate;
    int nheads;         // 0: per-channel A (D, N); > 0: scalar A per head
    bool bf16;
    bool softplus;
    hipStream_t stream;
    // Per-channel A: pass 1 hands its step sizes (rounded to the I/O dtype) to
    // pass 3 through the workspace; false: pass 3 recomputes them from delta and
    // the workspace holds the chunk carries only.
    bool dt_handoff = true;
};

// Chunking of the sequence used by the scan for a given shape.
struct ScanPlan {
    int64_t chunk_len;   // tokens per chunk (multiple of 64)
    int64_t nchunks;     // ceil(L / chunk_len)
};

ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim);
// The state size the scan's kernels run a requested N with (N itself, or the
// next compiled size, the states above N padded with zeros; pad.hip), or 0 when
// no kernel can run it.
int64_t scan_kernel_dstate(int64_t dim, int64_t dstate, int nheads, bool bf16);
size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads, bool bf16,
                            bool dt_handoff = true);
bool scan_supported(int64_t dim, int64_t dstate, int nheads, bool bf16);
hipError_t launch_selective_scan(const ScanArgs& a);

// Backward of the per-channel scan (scan_bwd.hip).
struct ScanBwdArgs {
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
    void* du;
    void* ddelta;
    float* dA;
    void* dB;
    void* dC;
    float* dD;            // or null
    void* dz;             // null iff z is null
    float* ddelta_bias;   // or null
    const float* initial_state = nullptr;   // (B, D, N) state before token 0, or null
    const float* d_final_state = nullptr;   // (B, D, N) gradient at the final state, or null
    float* d_initial_state = nullptr;       // (B, D, N), written; needs initial_state
    void* ws;
    int64_t batch, seqlen, dim, dstate;
    int nheads = 0;       // > 0: scalar A per head (heads_bwd.hip)
    bool bf16;
    bool softplus;
    hipStream_t stream;
};

bool scan_bwd_supported(int64_t dstate, int nheads);
int64_t scan_bwd_kernel_dstate(int64_t dstate, int nheads);   // as scan_kernel_dstate, or 0

// Backward of the scalar-A heads scan (heads_bwd.hip): the state size its
// kernels run a requested N with (0: unsupported), their workspace, the launch.
int64_t heads_bwd_kernel_dstate(int64_t dim, int64_t dstate, int nheads);
size_t heads_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads);
hipError_t launch_heads_bwd(const ScanBwdArgs& a);
size_t scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool bf16);
hipError_t launch_selective_scan_bwd(const ScanBwdArgs& a);

// One-token decode steps (decode.hip).
struct ConvUpdateArgs {
    const void* x;          // (B, D)
    void* conv_state;       // (B, D, 3), I/O dtype: x_{t-3}, x_{t-2}, x_{t-1}
    const float* weight;    // (D, 4)
    const float* bias;      // (D,) or null
    const uint8_t* reset;   // (B,) or null
    void* out;              // (B, D)
    int64_t batch, dim;
    bool bf16;
    bool apply_silu;
    hipStream_t stream;
};

struct StateUpdateArgs {
    float* state;           // (B, D, N) float32, in place
    const void* u;          // (B, D)
    const void* delta;      // (B, D) or (B, H)
    const float* A;         // (D, N) or (H,)
    const void* B;          // (B, N)
    const void* C;          // (B, N)
    const float* D;
    const void* z;
    const float* delta_bias;
    const uint8_t* reset;   // (B,) or null
    void* out;              // (B, D)
    int64_t batch, dim, dstate;
    int nheads;
    bool bf16;
    bool softplus;
    hipStream_t stream;
    // Fused conv step (conv_x set): u is formed from conv_x and the window, which
    // is updated in place; u is also written to u_out when that is not null.
    const void* conv_x = nullptr;      // (B, D)
    void* conv_state = nullptr;        // (B, D, 3), I/O dtype
    const float* conv_w = nullptr;     // (D, 4)
    const float* conv_b = nullptr;     // (D,) or null
    void* u_out = nullptr;             // (B, D) or null
};

hipError_t launch_conv1d_update(const ConvUpdateArgs& a);
bool state_update_supported(int64_t dstate);
hipError_t launch_state_update(const StateUpdateArgs& a);

// Scalar-A heads with bf16 I/O: the chunked matrix-core form (ssd.hip).
bool ssd_supported(int64_t dim, int64_t dstate, int nheads);
size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int nheads);
hipError_t launch_ssd(const ScanArgs& a);

// Row padding of the state dimension (pad.hip): dst rows of nt elements from
// src rows of n (zeros above n), and back; esz is 2 or 4 bytes.
hipError_t launch_pad_rows(const void* src, void* dst, int64_t rows, int n, int nt, int esz, hipStream_t stream);
hipError_t launch_unpad_rows(const void* src, void* dst, int64_t rows, int n, int nt, int esz, hipStream_t stream);

// The library's own device scratch for callers that cannot allocate
// (noalloc.hip): its size, and its address on the device of `stream`.
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

}  // namespace mamba
