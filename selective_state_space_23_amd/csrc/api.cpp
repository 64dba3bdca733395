// C ABI of the Mamba selective-scan forward path: argument validation and
// dispatch to the HIP kernels.  Every check runs on the host before any launch,
// so an invalid call never reaches the GPU.
#include "mamba_hip.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "fill.hpp"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;        // channels per row
constexpr int64_t kMaxElems = int64_t(1) << 40;      // elements per tensor
constexpr int64_t kMaxSeqlen = 3000000;              // grid.y limits of the kernels

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap (null or empty ranges never do).
bool overlap(const void* p, size_t bytes, const void* q, size_t qbytes) {
    if (!p || !q || bytes == 0 || qbytes == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qbytes && b < a + bytes;
}

bool mul_ok(int64_t a, int64_t b, int64_t c, int64_t* out) {
    if (a < 0 || b < 0 || c < 0) return false;
    __int128 r = static_cast<__int128>(a) * b * c;
    if (r > kMaxElems) return false;
    *out = static_cast<int64_t>(r);
    return true;
}

int check_dims(const mamba_scan_dims_t* d) {
    if (!d) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d->batch < 0 || d->seqlen < 0 || d->dim < 0 || d->dstate < 1) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d->dim > kMaxDim || d->batch > 65535 || d->nheads < 0) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d->seqlen > kMaxSeqlen) return MAMBA_ERR_UNSUPPORTED;
    if (d->dtype != MAMBA_DTYPE_F32 && d->dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d->nheads > 0 && (d->dim % d->nheads) != 0) return MAMBA_ERR_INVALID_ARGUMENT;
    int64_t n;
    if (!mul_ok(d->batch, d->seqlen, d->dim, &n)) return MAMBA_ERR_INVALID_ARGUMENT;
    if (!mul_ok(d->batch, d->seqlen, d->dstate, &n)) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d->ngroups != 1) return MAMBA_ERR_UNSUPPORTED;
    // The scan kernels address one batch row of a tensor with 32-bit byte offsets
    // (up to 64 tokens past the row end, which read as zeros).
    const int64_t widest = d->dim > d->dstate ? d->dim : d->dstate;
    if ((d->seqlen + 64) * widest * 4 > INT32_MAX) return MAMBA_ERR_UNSUPPORTED;
    if (!mamba::scan_supported(d->dim, d->dstate, d->nheads, d->dtype == MAMBA_DTYPE_BF16)) return MAMBA_ERR_UNSUPPORTED;
    return MAMBA_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of one forward scan: the kernels' own workspace at the state size nt
// they run with, then, when nt > N, the zero-padded copies (pad.hip) of B, C, A
// and the initial and final states.
struct FwdLayout {
    int64_t n = 0, nt = 0;
    size_t off_B = 0, off_C = 0, off_A = 0, off_h0 = 0, off_hT = 0, total = 0;
    bool padded() const { return nt != n; }
};

FwdLayout fwd_layout(const mamba_scan_dims_t* d, bool dt_handoff) {
    FwdLayout w;
    const bool bf16 = d->dtype == MAMBA_DTYPE_BF16;
    w.n = d->dstate;
    w.nt = mamba::scan_kernel_dstate(d->dim, d->dstate, d->nheads, bf16);
    size_t off = mamba::scan_workspace_bytes(d->batch, d->seqlen, d->dim, w.nt, d->nheads, bf16, dt_handoff);
    if (!w.padded()) {
        w.total = off;
        return w;
    }
    const size_t esz = bf16 ? 2 : 4;
    const size_t bc = static_cast<size_t>(d->batch * d->seqlen * w.nt) * esz;
    const size_t st = static_cast<size_t>(d->batch * d->dim * w.nt) * 4;
    off = align256(off);
    w.off_B = off; off += align256(bc);
    w.off_C = off; off += align256(bc);
    w.off_A = off; off += d->nheads ? 0 : align256(static_cast<size_t>(d->dim * w.nt) * 4);
    w.off_h0 = off; off += align256(st);
    w.off_hT = off; off += align256(st);
    w.total = off;
    return w;
}

// Runs the scan of `a` (whose dstate is the requested N), on zero-padded copies
// in the workspace when the kernels run a larger state size.
hipError_t launch_scan_layout(mamba::ScanArgs a, const FwdLayout& w) {
    if (!w.padded()) return mamba::launch_selective_scan(a);
    char* ws = reinterpret_cast<char*>(a.ws);
    const int esz = a.bf16 ? 2 : 4;
    const int n = static_cast<int>(w.n), nt = static_cast<int>(w.nt);
    const int64_t bl = a.batch * a.seqlen, bd = a.batch * a.dim;
    hipError_t e;
    if ((e = mamba::launch_pad_rows(a.B, ws + w.off_B, bl, n, nt, esz, a.stream)) != hipSuccess) return e;
    if ((e = mamba::launch_pad_rows(a.C, ws + w.off_C, bl, n, nt, esz, a.stream)) != hipSuccess) return e;
    if (a.nheads == 0 && (e = mamba::launch_pad_rows(a.A, ws + w.off_A, a.dim, n, nt, 4, a.stream)) != hipSuccess)
        return e;
    if (a.initial_state &&
        (e = mamba::launch_pad_rows(a.initial_state, ws + w.off_h0, bd, n, nt, 4, a.stream)) != hipSuccess)
        return e;
    float* fin = a.final_state;
    a.B = ws + w.off_B;
    a.C = ws + w.off_C;
    if (a.nheads == 0) a.A = reinterpret_cast<const float*>(ws + w.off_A);
    if (a.initial_state) a.initial_state = reinterpret_cast<const float*>(ws + w.off_h0);
    a.final_state = fin ? reinterpret_cast<float*>(ws + w.off_hT) : nullptr;
    a.dstate = nt;
    if ((e = mamba::launch_selective_scan(a)) != hipSuccess) return e;
    return fin ? mamba::launch_unpad_rows(ws + w.off_hT, fin, bd, n, nt, 4, a.stream) : hipSuccess;
}

// Workspace of one scan backward: the kernels' own workspace at their state size
// nt, then, when nt > N, zero-padded copies of B, C, A, the initial state and the
// final state's gradient, and the padded gradients dA, dB, dC, d_initial_state
// whose first N states per row are copied out.
struct BwdLayout {
    int64_t n = 0, nt = 0;
    size_t off_B = 0, off_C = 0, off_A = 0, off_h0 = 0, off_dhT = 0;
    size_t off_dA = 0, off_dB = 0, off_dC = 0, off_dh0 = 0, total = 0;
    bool padded() const { return nt != n; }
};

// The backward's kernels: per-channel A (scan_bwd.hip) or scalar-A heads
// (heads_bwd.hip); the state size they run N with (0: unsupported).
int64_t bwd_kernel_dstate(const mamba_scan_dims_t* d) {
    return d->nheads > 0 ? mamba::heads_bwd_kernel_dstate(d->dim, d->dstate, d->nheads)
                         : mamba::scan_bwd_kernel_dstate(d->dstate, 0);
}

BwdLayout bwd_layout_of(const mamba_scan_dims_t* d) {
    BwdLayout w;
    const bool bf16 = d->dtype == MAMBA_DTYPE_BF16;
    w.n = d->dstate;
    w.nt = bwd_kernel_dstate(d);
    size_t off = d->nheads > 0 ? mamba::heads_bwd_workspace_bytes(d->batch, d->seqlen, d->dim, w.nt, d->nheads)
                               : mamba::scan_bwd_workspace_bytes(d->batch, d->seqlen, d->dim, w.nt, bf16);
    if (!w.padded()) {
        w.total = off;
        return w;
    }
    const size_t esz = bf16 ? 2 : 4;
    const size_t bc = align256(static_cast<size_t>(d->batch * d->seqlen * w.nt) * esz);
    const size_t st = align256(static_cast<size_t>(d->batch * d->dim * w.nt) * 4);
    // A and dA are (H,) for heads: nothing to pad
    const size_t dn = d->nheads > 0 ? 0 : align256(static_cast<size_t>(d->dim * w.nt) * 4);
    off = align256(off);
    w.off_B = off; off += bc;
    w.off_C = off; off += bc;
    w.off_A = off; off += dn;
    w.off_h0 = off; off += st;
    w.off_dhT = off; off += st;
    w.off_dA = off; off += dn;
    w.off_dB = off; off += bc;
    w.off_dC = off; off += bc;
    w.off_dh0 = off; off += st;
    w.total = off;
    return w;
}

hipError_t launch_bwd_kernels(const mamba::ScanBwdArgs& a) {
    return a.nheads > 0 ? mamba::launch_heads_bwd(a) : mamba::launch_selective_scan_bwd(a);
}

hipError_t launch_bwd_layout(mamba::ScanBwdArgs a, const BwdLayout& w) {
    if (!w.padded()) return launch_bwd_kernels(a);
    const bool heads = a.nheads > 0;
    char* ws = static_cast<char*>(a.ws);
    const int esz = a.bf16 ? 2 : 4;
    const int n = static_cast<int>(w.n), nt = static_cast<int>(w.nt);
    const int64_t bl = a.batch * a.seqlen, bd = a.batch * a.dim;
    const hipStream_t s = a.stream;
    hipError_t e;
    if ((e = mamba::launch_pad_rows(a.B, ws + w.off_B, bl, n, nt, esz, s)) != hipSuccess) return e;
    if ((e = mamba::launch_pad_rows(a.C, ws + w.off_C, bl, n, nt, esz, s)) != hipSuccess) return e;
    if (!heads && (e = mamba::launch_pad_rows(a.A, ws + w.off_A, a.dim, n, nt, 4, s)) != hipSuccess) return e;
    if (a.initial_state && (e = mamba::launch_pad_rows(a.initial_state, ws + w.off_h0, bd, n, nt, 4, s)) != hipSuccess)
        return e;
    if (a.d_final_state && (e = mamba::launch_pad_rows(a.d_final_state, ws + w.off_dhT, bd, n, nt, 4, s)) != hipSuccess)
        return e;
    float* dA = a.dA;
    void* dB = a.dB;
    void* dC = a.dC;
    float* dh0 = a.d_initial_state;
    a.B = ws + w.off_B;
    a.C = ws + w.off_C;
    if (!heads) a.A = reinterpret_cast<const float*>(ws + w.off_A);
    if (a.initial_state) a.initial_state = reinterpret_cast<const float*>(ws + w.off_h0);
    if (a.d_final_state) a.d_final_state = reinterpret_cast<const float*>(ws + w.off_dhT);
    if (!heads) a.dA = reinterpret_cast<float*>(ws + w.off_dA);
    a.dB = ws + w.off_dB;
    a.dC = ws + w.off_dC;
    if (dh0) a.d_initial_state = reinterpret_cast<float*>(ws + w.off_dh0);
    a.dstate = nt;
    if ((e = launch_bwd_kernels(a)) != hipSuccess) return e;
    if (!heads && (e = mamba::launch_unpad_rows(ws + w.off_dA, dA, a.dim, n, nt, 4, s)) != hipSuccess) return e;
    if ((e = mamba::launch_unpad_rows(ws + w.off_dB, dB, bl, n, nt, esz, s)) != hipSuccess) return e;
    if ((e = mamba::launch_unpad_rows(ws + w.off_dC, dC, bl, n, nt, esz, s)) != hipSuccess) return e;
    return dh0 ? mamba::launch_unpad_rows(ws + w.off_dh0, dh0, bd, n, nt, 4, s) : hipSuccess;
}

// Checks of one conv1d call (shared by the conv and the fused conv + scan entry
// points); fills `a` on success.
int check_conv(const void* x, const float* weight, const float* bias, const uint8_t* doc_start,
               const void* conv_state, void* out, int64_t batch, int64_t seqlen, int64_t dim, int32_t width,
               int32_t dtype, int32_t apply_silu, void* stream, mamba::ConvArgs* a, bool* empty,
               bool out_optional = false) {
    *empty = false;
    if (batch < 0 || seqlen < 0 || dim < 0) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARGUMENT;
    if (width != 4) return MAMBA_ERR_UNSUPPORTED;
    int64_t n;
    if (!mul_ok(batch, seqlen, dim, &n) || dim > kMaxDim || batch > 65535) return MAMBA_ERR_INVALID_ARGUMENT;
    if (seqlen > kMaxSeqlen) return MAMBA_ERR_UNSUPPORTED;
    if (n == 0) {
        *empty = true;
        return MAMBA_OK;
    }
    if (!x || !weight || (!out && !out_optional)) return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(x, esz) || (out && !aligned(out, esz)) || !aligned(weight, 4) || (bias && !aligned(bias, 4)) ||
        (conv_state && !aligned(conv_state, esz)))
        return MAMBA_ERR_MISALIGNED;
    const size_t bytes = static_cast<size_t>(n) * esz;
    const size_t hist = static_cast<size_t>(batch * dim * 3) * esz;
    if (overlap(x, bytes, out, bytes) || overlap(weight, dim * 16, out, bytes) ||
        overlap(bias, dim * 4, out, bytes) || overlap(doc_start, batch * seqlen, out, bytes) ||
        overlap(conv_state, hist, out, bytes))
        return MAMBA_ERR_INVALID_ARGUMENT;

    a->x = x; a->weight = weight; a->bias = bias; a->doc_start = doc_start; a->conv_state = conv_state;
    a->out = out;
    a->batch = batch; a->seqlen = seqlen; a->dim = dim;
    a->bf16 = dtype == MAMBA_DTYPE_BF16;
    const int64_t vec = a->bf16 ? 8 : 4;
    a->vectorized = (dim % vec) == 0 && aligned(x, 16) && (!out || aligned(out, 16));
    a->apply_silu = apply_silu != 0;
    a->stream = static_cast<hipStream_t>(stream);
    return MAMBA_OK;
}

// Checks of one selective-scan call (shared by the scan and the fused conv + scan
// entry points); fills `a` on success.  For the fused call (nextra > 0) u is
// written too unless u_written is false (then `u` is the conv input, read only),
// and `extra` lists its further read-only inputs (conv input, weights, history;
// byte sizes in extra_sz): neither may overlap what else the call reads or
// writes.
int check_scan(const mamba_scan_dims_t* dims, const void* u, const void* delta, const float* A, const void* B,
               const void* C, const float* D, const void* z, const float* delta_bias, const uint8_t* doc_start,
               const float* initial_state, void* out, float* final_state, void* workspace, size_t workspace_bytes,
               void* stream, const void* const* extra, const size_t* extra_sz, int nextra, mamba::ScanArgs* a,
               FwdLayout* lay, bool* empty, bool own_scratch = false, bool u_written = true) {
    *empty = false;
    const int st = check_dims(dims);
    if (st != MAMBA_OK) return st;
    *lay = fwd_layout(dims, !own_scratch);
    const int64_t Bt = dims->batch, L = dims->seqlen, Dm = dims->dim, N = dims->dstate;
    if (Bt * L * Dm == 0) {
        *empty = true;
        return MAMBA_OK;
    }
    if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dims->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    const int64_t nd = dims->nheads ? dims->nheads : Dm;
    if (!aligned(u, esz) || !aligned(delta, esz) || !aligned(out, esz) || (z && !aligned(z, esz)))
        return MAMBA_ERR_MISALIGNED;
    // B and C rows are read as 32-bit words (element by element when padded).
    if (!aligned(B, esz) || !aligned(C, esz)) return MAMBA_ERR_MISALIGNED;
    if (!lay->padded() && (!aligned(B, 4) || !aligned(C, 4) || (N * esz) % 4 != 0)) return MAMBA_ERR_MISALIGNED;
    // Scalar-A heads with bf16 I/O move u, z, out, B and C in 16-byte vectors.
    if (dims->nheads > 0 && dims->dtype == MAMBA_DTYPE_BF16 &&
        (!aligned(u, 16) || !aligned(out, 16) || (z && !aligned(z, 16)) ||
         (!lay->padded() && (!aligned(B, 16) || !aligned(C, 16)))))
        return MAMBA_ERR_MISALIGNED;
    if (!aligned(A, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)) ||
        (final_state && !aligned(final_state, 4)) || (initial_state && !aligned(initial_state, 4)))
        return MAMBA_ERR_MISALIGNED;

    const size_t act = static_cast<size_t>(Bt * L * Dm) * esz;
    const size_t dlt = static_cast<size_t>(Bt * L * nd) * esz;
    const size_t bc = static_cast<size_t>(Bt * L * N) * esz;
    const size_t fsb = static_cast<size_t>(Bt * Dm * N) * 4;
    const size_t abytes = static_cast<size_t>(dims->nheads ? dims->nheads : Dm * N) * 4;
    const void* ins[] = {u, delta, B, C, z, A, D, delta_bias, doc_start, initial_state};
    const size_t insz[] = {act, dlt, bc, bc, act, abytes, static_cast<size_t>(Dm) * 4,
                           static_cast<size_t>(nd) * 4, static_cast<size_t>(Bt * L), fsb};
    constexpr int kIns = 10;
    for (int i = 0; i < kIns; ++i) {
        if (overlap(ins[i], insz[i], out, act)) return MAMBA_ERR_INVALID_ARGUMENT;
        if (overlap(ins[i], insz[i], final_state, fsb)) return MAMBA_ERR_INVALID_ARGUMENT;
    }
    if (overlap(out, act, final_state, fsb)) return MAMBA_ERR_INVALID_ARGUMENT;
    if (nextra > 0) {
        for (int i = 1; i < kIns && u_written; ++i)   // u is written: it may not overlap the scan's inputs
            if (overlap(ins[i], insz[i], u, act)) return MAMBA_ERR_INVALID_ARGUMENT;
        for (int i = 0; i < nextra; ++i)
            if (overlap(extra[i], extra_sz[i], out, act) || overlap(extra[i], extra_sz[i], final_state, fsb))
                return MAMBA_ERR_INVALID_ARGUMENT;
    }

    const size_t need = lay->total;
    if (own_scratch) {
        // The library's own scratch: a distinct device allocation of fixed size.
        if (need > mamba::noalloc_scratch_bytes()) return MAMBA_ERR_WORKSPACE;
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need) return MAMBA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return MAMBA_ERR_MISALIGNED;
        for (int i = 0; i < kIns; ++i)
            if (overlap(ins[i], insz[i], workspace, need)) return MAMBA_ERR_INVALID_ARGUMENT;
        if (overlap(out, act, workspace, need) || overlap(final_state, fsb, workspace, need))
            return MAMBA_ERR_INVALID_ARGUMENT;
        for (int i = 0; i < nextra; ++i)
            if (overlap(extra[i], extra_sz[i], workspace, need)) return MAMBA_ERR_INVALID_ARGUMENT;
    }

    a->u = u; a->delta = delta; a->A = A; a->B = B; a->C = C; a->D = D; a->z = z;
    a->delta_bias = delta_bias; a->doc_start = doc_start; a->initial_state = initial_state;
    a->out = out; a->final_state = final_state;
    a->ws = static_cast<float*>(workspace);
    a->batch = Bt; a->seqlen = L; a->dim = Dm; a->dstate = N;
    a->nheads = dims->nheads;
    a->bf16 = dims->dtype == MAMBA_DTYPE_BF16;
    a->softplus = dims->delta_softplus != 0;
    a->stream = static_cast<hipStream_t>(stream);
    a->dt_handoff = !own_scratch;
    return MAMBA_OK;
}

// Outputs of a call with no tokens (B L D == 0, dims already checked): the
// state passes through unchanged, final_state = initial_state (or 0).
int empty_scan_outputs(const mamba_scan_dims_t* dims, const float* initial_state, float* final_state,
                       void* stream) {
    const int64_t n = dims->batch * dims->dim * dims->dstate;
    if (dims->seqlen != 0 || n == 0 || final_state == nullptr) return MAMBA_OK;
    if (!aligned(final_state, 4) || (initial_state && !aligned(initial_state, 4))) return MAMBA_ERR_MISALIGNED;
    if (overlap(final_state, n * 4, initial_state, n * 4)) return MAMBA_ERR_INVALID_ARGUMENT;
    return mamba::launch_fill(final_state, initial_state, n, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MAMBA_OK
               : MAMBA_ERR_HIP;
}

// Zero-fills the float32 arrays (dst[i], n[i] elements) that are not null.
int zero_outputs(float* const* dst, const int64_t* n, int count, void* stream) {
    for (int i = 0; i < count; ++i)
        if (dst[i] && n[i] > 0 && !aligned(dst[i], 4)) return MAMBA_ERR_MISALIGNED;
    for (int i = 0; i < count; ++i)
        if (dst[i] && n[i] > 0 && mamba::launch_fill(dst[i], nullptr, n[i], static_cast<hipStream_t>(stream)) != hipSuccess)
            return MAMBA_ERR_HIP;
    return MAMBA_OK;
}

}  // namespace

extern "C" {

int mamba_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* mamba_status_string(int status) {
    switch (status) {
        case MAMBA_OK: return "ok";
        case MAMBA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MAMBA_ERR_UNSUPPORTED: return "unsupported configuration";
        case MAMBA_ERR_MISALIGNED: return "misaligned pointer";
        case MAMBA_ERR_WORKSPACE: return "workspace missing or too small";
        case MAMBA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int mamba_causal_conv1d_fwd(const void* x, const float* weight, const float* bias, const uint8_t* doc_start,
                            const void* conv_state, void* out, int64_t batch, int64_t seqlen, int64_t dim,
                            int32_t width, int32_t dtype, int32_t apply_silu, void* stream) {
    mamba::ConvArgs a;
    bool empty;
    const int st = check_conv(x, weight, bias, doc_start, conv_state, out, batch, seqlen, dim, width, dtype,
                              apply_silu, stream, &a, &empty);
    if (st != MAMBA_OK || empty) return st;
    return mamba::launch_causal_conv1d(a) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}


int mamba_selective_scan_workspace_bytes(const mamba_scan_dims_t* dims, size_t* bytes) {
    if (!bytes) return MAMBA_ERR_INVALID_ARGUMENT;
    *bytes = 0;
    const int st = check_dims(dims);
    if (st != MAMBA_OK) return st;
    *bytes = fwd_layout(dims, true).total;
    return MAMBA_OK;
}

int mamba_selective_scan_fwd(const mamba_scan_dims_t* dims, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, const uint8_t* doc_start, const float* initial_state,
                             void* out, float* final_state, void* workspace, size_t workspace_bytes,
                             void* stream) {
    mamba::ScanArgs a;
    FwdLayout lay;
    bool empty;
    const int st = check_scan(dims, u, delta, A, B, C, D, z, delta_bias, doc_start, initial_state, out,
                              final_state, workspace, workspace_bytes, stream, nullptr, nullptr, 0, &a, &lay, &empty);
    if (st != MAMBA_OK) return st;
    if (empty) return empty_scan_outputs(dims, initial_state, final_state, stream);
    return launch_scan_layout(a, lay) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_selective_scan_fwd_noalloc(const mamba_scan_dims_t* dims, const void* u, const void* delta,
                                     const float* A, const void* B, const void* C, const float* D, const void* z,
                                     const float* delta_bias, const uint8_t* doc_start, const float* initial_state,
                                     void* out, float* final_state, void* stream) {
    mamba::ScanArgs a;
    FwdLayout lay;
    bool empty;
    const int st = check_scan(dims, u, delta, A, B, C, D, z, delta_bias, doc_start, initial_state, out,
                              final_state, nullptr, 0, stream, nullptr, nullptr, 0, &a, &lay, &empty, true);
    if (st != MAMBA_OK) return st;
    if (empty) return empty_scan_outputs(dims, initial_state, final_state, stream);
    void* ws = nullptr;
    if (mamba::noalloc_scratch(a.stream, &ws) != hipSuccess) return MAMBA_ERR_HIP;
    a.ws = static_cast<float*>(ws);
    return launch_scan_layout(a, lay) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_conv_scan_fwd(const mamba_scan_dims_t* dims, const void* x, const float* conv_weight,
                        const float* conv_bias, const void* conv_state, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                        const uint8_t* doc_start, const float* initial_state, void* u, void* out, float* final_state,
                        void* workspace, size_t workspace_bytes, void* stream) {
    const int sd = check_dims(dims);
    if (sd != MAMBA_OK) return sd;
    mamba::ConvArgs ca;
    bool empty;
    const bool has_u = u != nullptr;        // NULL: the conv output is not written
    int st = check_conv(x, conv_weight, conv_bias, doc_start, conv_state, u, dims->batch, dims->seqlen, dims->dim, 4,
                        dims->dtype, 1, stream, &ca, &empty, true);
    if (st != MAMBA_OK) return st;
    if (empty) return empty_scan_outputs(dims, initial_state, final_state, stream);
    // Per-channel A: the conv runs inside the scan's first pass.  bf16 scalar-A
    // heads: the conv kernel writes u first (faster than forming u in the
    // matrix-form passes), unless there is no u; then both passes form it.  The
    // fp32 recurrent form of heads always runs the conv kernel first: it needs u.
    const bool heads_bf16 = dims->nheads > 0 && dims->dtype == MAMBA_DTYPE_BF16;
    const bool fused_conv = dims->nheads == 0 || (heads_bf16 && !has_u);
    if (!has_u && !fused_conv) return MAMBA_ERR_UNSUPPORTED;
    // The bf16 heads scan reads its conv input in 16-byte vectors, as it reads u.
    if (heads_bf16 && !has_u && !aligned(x, 16)) return MAMBA_ERR_MISALIGNED;
    // u is written by the conv and read by the scan: it may overlap nothing else.
    const size_t esz = dims->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    const size_t act = static_cast<size_t>(dims->batch * dims->seqlen * dims->dim) * esz;
    const void* conv_in[] = {x, conv_weight, conv_bias, conv_state};
    const size_t conv_sz[] = {act, static_cast<size_t>(dims->dim) * 16, static_cast<size_t>(dims->dim) * 4,
                              static_cast<size_t>(dims->batch * dims->dim * 3) * esz};
    mamba::ScanArgs a;
    FwdLayout lay;
    st = check_scan(dims, has_u ? u : x, delta, A, B, C, D, z, delta_bias, doc_start, initial_state, out, final_state,
                    workspace, workspace_bytes, stream, conv_in, conv_sz, 4, &a, &lay, &empty, false, has_u);
    if (st != MAMBA_OK) return st;
    if (empty) return empty_scan_outputs(dims, initial_state, final_state, stream);
    if (fused_conv) {
        a.conv_x = x; a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state = conv_state;
        a.u = u;                    // the conv output's destination, or NULL
        return launch_scan_layout(a, lay) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
    }
    if (mamba::launch_causal_conv1d(ca) != hipSuccess) return MAMBA_ERR_HIP;
    return launch_scan_layout(a, lay) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_causal_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, size_t* bytes) {
    if (!bytes) return MAMBA_ERR_INVALID_ARGUMENT;
    *bytes = 0;
    int64_t n;
    if (!mul_ok(batch, seqlen, dim, &n) || dim > kMaxDim || batch > 65535) return MAMBA_ERR_INVALID_ARGUMENT;
    if (seqlen > kMaxSeqlen) return MAMBA_ERR_UNSUPPORTED;
    *bytes = mamba::conv_bwd_workspace_bytes(batch, seqlen, dim);
    return MAMBA_OK;
}

int mamba_causal_conv1d_bwd(const void* x, const float* weight, const float* bias, const uint8_t* doc_start,
                            const void* conv_state, const void* du, void* dx, float* dweight, float* dbias,
                            float* d_conv_state, int64_t batch, int64_t seqlen, int64_t dim, int32_t width,
                            int32_t dtype, int32_t apply_silu, void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 0 || seqlen < 0 || dim < 0) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARGUMENT;
    if (width != 4) return MAMBA_ERR_UNSUPPORTED;
    int64_t n;
    if (!mul_ok(batch, seqlen, dim, &n) || dim > kMaxDim || batch > 65535) return MAMBA_ERR_INVALID_ARGUMENT;
    if (seqlen > kMaxSeqlen) return MAMBA_ERR_UNSUPPORTED;
    if (d_conv_state && !conv_state) return MAMBA_ERR_INVALID_ARGUMENT;
    if (n == 0) {
        // No tokens: the weight and bias gradients are sums over none, and the
        // history influenced nothing.
        float* zs[] = {batch * seqlen == 0 ? dweight : nullptr, batch * seqlen == 0 ? dbias : nullptr,
                       seqlen == 0 ? d_conv_state : nullptr};
        const int64_t zn[] = {dim * 4, dim, batch * dim * 3};
        return zero_outputs(zs, zn, 3, stream);
    }
    if (!x || !weight || !du || !dx || !dweight) return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(du, esz) || !aligned(dx, esz) || !aligned(weight, 4) || !aligned(dweight, 4) ||
        (bias && !aligned(bias, 4)) || (dbias && !aligned(dbias, 4)) || (conv_state && !aligned(conv_state, esz)) ||
        (d_conv_state && !aligned(d_conv_state, 4)))
        return MAMBA_ERR_MISALIGNED;
    const size_t act = static_cast<size_t>(n) * esz;
    const size_t hist = static_cast<size_t>(batch * dim * 3);
    const size_t need = mamba::conv_bwd_workspace_bytes(batch, seqlen, dim);
    if (!workspace || workspace_bytes < need) return MAMBA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MAMBA_ERR_MISALIGNED;
    const void* ins[] = {x, weight, bias, doc_start, du, conv_state};
    const size_t insz[] = {act, static_cast<size_t>(dim) * 16, static_cast<size_t>(dim) * 4,
                           static_cast<size_t>(batch * seqlen), act, hist * esz};
    const void* outs[] = {dx, dweight, dbias, d_conv_state, workspace};
    const size_t outsz[] = {act, static_cast<size_t>(dim) * 16, static_cast<size_t>(dim) * 4, hist * 4, need};
    for (int o = 0; o < 5; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[o], outsz[o], ins[i], insz[i])) return MAMBA_ERR_INVALID_ARGUMENT;
        for (int k = o + 1; k < 5; ++k)
            if (overlap(outs[o], outsz[o], outs[k], outsz[k])) return MAMBA_ERR_INVALID_ARGUMENT;
    }
    mamba::ConvBwdArgs a;
    a.x = x; a.weight = weight; a.bias = bias; a.doc_start = doc_start; a.du = du; a.dx = dx;
    a.dweight = dweight; a.dbias = dbias; a.ws = static_cast<float*>(workspace);
    a.conv_state = conv_state; a.d_conv_state = d_conv_state;
    a.batch = batch; a.seqlen = seqlen; a.dim = dim;
    a.bf16 = dtype == MAMBA_DTYPE_BF16;
    const size_t vbytes = 2 * esz;           // channel pairs
    a.vectorized = (dim % 2) == 0 && aligned(x, vbytes) && aligned(du, vbytes) && aligned(dx, vbytes);
    a.apply_silu = apply_silu != 0;
    a.stream = static_cast<hipStream_t>(stream);
    return mamba::launch_causal_conv1d_bwd(a) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_selective_scan_bwd_workspace_bytes(const mamba_scan_dims_t* dims, size_t* bytes) {
    if (!bytes) return MAMBA_ERR_INVALID_ARGUMENT;
    *bytes = 0;
    const int st = check_dims(dims);
    if (st != MAMBA_OK) return st;
    if (bwd_kernel_dstate(dims) == 0) return MAMBA_ERR_UNSUPPORTED;
    *bytes = bwd_layout_of(dims).total;
    return MAMBA_OK;
}

int mamba_selective_scan_bwd(const mamba_scan_dims_t* dims, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                             const uint8_t* doc_start, const float* initial_state, const void* dout,
                             const float* d_final_state, void* du, void* ddelta, float* dA, void* dB, void* dC,
                             float* dD, void* dz, float* ddelta_bias, float* d_initial_state, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const int st = check_dims(dims);
    if (st != MAMBA_OK) return st;
    if (bwd_kernel_dstate(dims) == 0) return MAMBA_ERR_UNSUPPORTED;
    const int64_t Bt = dims->batch, L = dims->seqlen, Dm = dims->dim, N = dims->dstate;
    const bool heads = dims->nheads > 0;
    const int64_t nd = heads ? dims->nheads : Dm;          // width of delta, ddelta, delta_bias, ddelta_bias
    const int64_t na = heads ? dims->nheads : Dm * N;      // elements of A and dA
    if ((z == nullptr) != (dz == nullptr)) return MAMBA_ERR_INVALID_ARGUMENT;
    if (d_initial_state && !initial_state) return MAMBA_ERR_INVALID_ARGUMENT;
    if (Bt * L * Dm == 0) {
        // No tokens: dA, dD and ddelta_bias are sums over none, and the adjoint
        // passes through the empty row (d_initial_state = d_final_state, or 0).
        float* zs[] = {Bt * L == 0 ? dA : nullptr, Bt * L == 0 ? dD : nullptr, Bt * L == 0 ? ddelta_bias : nullptr};
        const int64_t zn[] = {na, Dm, nd};
        int zst = zero_outputs(zs, zn, 3, stream);
        if (zst != MAMBA_OK || L != 0 || Bt * Dm == 0 || !d_initial_state) return zst;
        const int64_t ns = Bt * Dm * N;
        if (!aligned(d_initial_state, 4) || (d_final_state && !aligned(d_final_state, 4))) return MAMBA_ERR_MISALIGNED;
        if (overlap(d_initial_state, ns * 4, d_final_state, ns * 4)) return MAMBA_ERR_INVALID_ARGUMENT;
        return mamba::launch_fill(d_initial_state, d_final_state, ns, static_cast<hipStream_t>(stream)) == hipSuccess
                   ? MAMBA_OK
                   : MAMBA_ERR_HIP;
    }
    if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
        return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dims->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    // The per-channel main pass stages u, delta, z and dout through 4-byte loads
    // (pairs of bf16 channels): even D, 4-byte aligned rows.
    if (!heads && esz == 2 && Dm % 2 != 0) return MAMBA_ERR_UNSUPPORTED;
    const void* staged[] = {u, delta, z, dout};
    for (const void* t : staged)
        if (t && !aligned(t, 4)) return MAMBA_ERR_MISALIGNED;
    const void* acts[] = {du, ddelta, dz};
    for (const void* t : acts)
        if (t && !aligned(t, esz)) return MAMBA_ERR_MISALIGNED;
    const BwdLayout lay = bwd_layout_of(dims);
    if (!aligned(B, esz) || !aligned(C, esz) || !aligned(dB, esz) || !aligned(dC, esz)) return MAMBA_ERR_MISALIGNED;
    if (!lay.padded() && (!aligned(B, 4) || !aligned(C, 4) || (N * esz) % 4 != 0)) return MAMBA_ERR_MISALIGNED;
    const float* f32s[] = {A, D, delta_bias, dA, dD, ddelta_bias, initial_state, d_final_state, d_initial_state};
    for (const float* t : f32s)
        if (t && !aligned(t, 4)) return MAMBA_ERR_MISALIGNED;

    const size_t act = static_cast<size_t>(Bt * L * Dm) * esz;
    const size_t dlt = static_cast<size_t>(Bt * L * nd) * esz;
    const size_t bc = static_cast<size_t>(Bt * L * N) * esz;
    const size_t dn = static_cast<size_t>(na) * 4, d1 = static_cast<size_t>(Dm) * 4;
    const size_t n1 = static_cast<size_t>(nd) * 4;
    const size_t sb = static_cast<size_t>(Bt * Dm * N) * 4;
    const void* ins[] = {u, delta, A, B, C, D, z, delta_bias, doc_start, dout, initial_state, d_final_state};
    const size_t insz[] = {act, dlt, dn, bc, bc, d1, act, n1, static_cast<size_t>(Bt * L), act, sb, sb};
    constexpr int kIns = 12;
    const void* outs[] = {du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, d_initial_state};
    const size_t outsz[] = {act, dlt, dn, bc, bc, d1, act, n1, sb};
    constexpr int kOuts = 9;
    const size_t need = lay.total;
    if (!workspace || workspace_bytes < need) return MAMBA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MAMBA_ERR_MISALIGNED;
    for (int o = 0; o < kOuts; ++o) {
        for (int i = 0; i < kIns; ++i)
            if (overlap(outs[o], outsz[o], ins[i], insz[i])) return MAMBA_ERR_INVALID_ARGUMENT;
        for (int k = o + 1; k < kOuts; ++k)
            if (overlap(outs[o], outsz[o], outs[k], outsz[k])) return MAMBA_ERR_INVALID_ARGUMENT;
        if (overlap(outs[o], outsz[o], workspace, need)) return MAMBA_ERR_INVALID_ARGUMENT;
    }
    for (int i = 0; i < kIns; ++i)
        if (overlap(ins[i], insz[i], workspace, need)) return MAMBA_ERR_INVALID_ARGUMENT;

    mamba::ScanBwdArgs a;
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.delta_bias = delta_bias;
    a.doc_start = doc_start; a.dout = dout;
    a.initial_state = initial_state; a.d_final_state = d_final_state; a.d_initial_state = d_initial_state;
    a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dz = dz; a.ddelta_bias = ddelta_bias;
    a.ws = workspace;
    a.batch = Bt; a.seqlen = L; a.dim = Dm; a.dstate = N;
    a.nheads = dims->nheads;
    a.bf16 = dims->dtype == MAMBA_DTYPE_BF16;
    a.softplus = dims->delta_softplus != 0;
    a.stream = static_cast<hipStream_t>(stream);
    return launch_bwd_layout(a, lay) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_causal_conv1d_update(const void* x, void* conv_state, const float* weight, const float* bias,
                               const uint8_t* reset, void* out, int64_t batch, int64_t dim, int32_t width,
                               int32_t dtype, int32_t apply_silu, void* stream) {
    if (batch < 0 || dim < 0 || batch > 65535 || dim > kMaxDim) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARGUMENT;
    if (width != 4) return MAMBA_ERR_UNSUPPORTED;
    if (batch * dim == 0) return MAMBA_OK;
    if (!x || !conv_state || !weight || !out) return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(conv_state, esz) || !aligned(out, esz) || !aligned(weight, 4) ||
        (bias && !aligned(bias, 4)))
        return MAMBA_ERR_MISALIGNED;
    const size_t act = static_cast<size_t>(batch * dim) * esz;
    if (overlap(x, act, out, act) || overlap(conv_state, act * 3, out, act) || overlap(x, act, conv_state, act * 3) ||
        overlap(weight, dim * 16, out, act) || overlap(bias, dim * 4, out, act) ||
        overlap(reset, batch, out, act) || overlap(weight, dim * 16, conv_state, act * 3))
        return MAMBA_ERR_INVALID_ARGUMENT;
    mamba::ConvUpdateArgs a;
    a.x = x; a.conv_state = conv_state; a.weight = weight; a.bias = bias; a.reset = reset; a.out = out;
    a.batch = batch; a.dim = dim;
    a.bf16 = dtype == MAMBA_DTYPE_BF16;
    a.apply_silu = apply_silu != 0;
    a.stream = static_cast<hipStream_t>(stream);
    return mamba::launch_conv1d_update(a) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // extern "C"

namespace {

// Checks of one decode recurrence step (shared by the plain and the fused entry
// points); `u` is the step's input (x for the fused step).  Fills `a`.
int check_state_update(const mamba_scan_dims_t* dims, float* state, const void* u, const void* delta, const float* A,
                       const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                       const uint8_t* reset, void* out, void* stream, mamba::StateUpdateArgs* a, bool* empty) {
    *empty = false;
    if (!dims) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dims->batch < 0 || dims->dim < 0 || dims->dstate < 1 || dims->nheads < 0 || dims->batch > 65535 ||
        dims->dim > kMaxDim || dims->seqlen != 1)
        return MAMBA_ERR_INVALID_ARGUMENT;
    if (dims->dtype != MAMBA_DTYPE_F32 && dims->dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dims->nheads > 0 && dims->dim % dims->nheads != 0) return MAMBA_ERR_INVALID_ARGUMENT;
    if (dims->ngroups != 1 || !mamba::state_update_supported(dims->dstate)) return MAMBA_ERR_UNSUPPORTED;
    const int64_t Bt = dims->batch, Dm = dims->dim, N = dims->dstate;
    if (Bt * Dm == 0) {
        *empty = true;
        return MAMBA_OK;
    }
    if (!state || !u || !delta || !A || !B || !C || !out) return MAMBA_ERR_INVALID_ARGUMENT;
    const size_t esz = dims->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    // A state row whose length is a power of two from 4 up is moved in 16-byte pieces.
    const bool pow2 = N >= 4 && (N & (N - 1)) == 0;
    if (!aligned(state, pow2 ? 16 : 4) || !aligned(u, esz) || !aligned(delta, esz) || !aligned(B, esz) ||
        !aligned(C, esz) ||
        !aligned(out, esz) || (z && !aligned(z, esz)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (delta_bias && !aligned(delta_bias, 4)))
        return MAMBA_ERR_MISALIGNED;
    const int64_t nd = dims->nheads ? dims->nheads : Dm;
    const size_t act = static_cast<size_t>(Bt * Dm) * esz;
    const size_t sb = static_cast<size_t>(Bt * Dm * N) * 4;
    const void* ins[] = {u, delta, A, B, C, D, z, delta_bias, reset};
    const size_t insz[] = {act, static_cast<size_t>(Bt * nd) * esz,
                           static_cast<size_t>(dims->nheads ? dims->nheads : Dm * N) * 4,
                           static_cast<size_t>(Bt * N) * esz, static_cast<size_t>(Bt * N) * esz,
                           static_cast<size_t>(Dm) * 4, act, static_cast<size_t>(nd) * 4, static_cast<size_t>(Bt)};
    for (int i = 0; i < 9; ++i)
        if (overlap(ins[i], insz[i], out, act) || overlap(ins[i], insz[i], state, sb)) return MAMBA_ERR_INVALID_ARGUMENT;
    if (overlap(out, act, state, sb)) return MAMBA_ERR_INVALID_ARGUMENT;
    a->state = state; a->u = u; a->delta = delta; a->A = A; a->B = B; a->C = C; a->D = D; a->z = z;
    a->delta_bias = delta_bias; a->reset = reset; a->out = out;
    a->batch = Bt; a->dim = Dm; a->dstate = N; a->nheads = dims->nheads;
    a->bf16 = dims->dtype == MAMBA_DTYPE_BF16;
    a->softplus = dims->delta_softplus != 0;
    a->stream = static_cast<hipStream_t>(stream);
    return MAMBA_OK;
}

}  // namespace

extern "C" {

int mamba_selective_state_update(const mamba_scan_dims_t* dims, float* state, const void* u, const void* delta,
                                 const float* A, const void* B, const void* C, const float* D, const void* z,
                                 const float* delta_bias, const uint8_t* reset, void* out, void* stream) {
    mamba::StateUpdateArgs a;
    bool empty;
    const int st = check_state_update(dims, state, u, delta, A, B, C, D, z, delta_bias, reset, out, stream, &a, &empty);
    if (st != MAMBA_OK || empty) return st;
    return mamba::launch_state_update(a) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_conv_state_update(const mamba_scan_dims_t* dims, const void* x, void* conv_state, const float* conv_weight,
                            const float* conv_bias, float* state, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* delta_bias,
                            const uint8_t* reset, void* u_out, void* out, void* stream) {
    mamba::StateUpdateArgs a;
    bool empty;
    const int st = check_state_update(dims, state, x, delta, A, B, C, D, z, delta_bias, reset, out, stream, &a, &empty);
    if (st != MAMBA_OK || empty) return st;
    if (!conv_state || !conv_weight) return MAMBA_ERR_INVALID_ARGUMENT;
    const int64_t Bt = dims->batch, Dm = dims->dim;
    const size_t esz = dims->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(conv_state, esz) || !aligned(conv_weight, 4) || (conv_bias && !aligned(conv_bias, 4)) ||
        (u_out && !aligned(u_out, esz)))
        return MAMBA_ERR_MISALIGNED;
    const size_t act = static_cast<size_t>(Bt * Dm) * esz;
    const size_t win = act * 3;
    const size_t sb = static_cast<size_t>(Bt * Dm * dims->dstate) * 4;
    // the window and u are written: neither may overlap anything else of the call
    const int64_t nd = dims->nheads ? dims->nheads : Dm;
    const void* others[] = {x, delta, A, B, C, D, z, delta_bias, reset, conv_weight, conv_bias, state, out};
    const size_t osz[] = {act, static_cast<size_t>(Bt * nd) * esz,
                          static_cast<size_t>(dims->nheads ? dims->nheads : Dm * dims->dstate) * 4,
                          static_cast<size_t>(Bt * dims->dstate) * esz, static_cast<size_t>(Bt * dims->dstate) * esz,
                          static_cast<size_t>(Dm) * 4, act, static_cast<size_t>(nd) * 4, static_cast<size_t>(Bt),
                          static_cast<size_t>(Dm) * 16, static_cast<size_t>(Dm) * 4, sb, act};
    for (int i = 0; i < 13; ++i)
        if (overlap(conv_state, win, others[i], osz[i]) || overlap(u_out, act, others[i], osz[i]))
            return MAMBA_ERR_INVALID_ARGUMENT;
    if (overlap(conv_state, win, u_out, act)) return MAMBA_ERR_INVALID_ARGUMENT;
    a.u = nullptr;
    a.conv_x = x; a.conv_state = conv_state; a.conv_w = conv_weight; a.conv_b = conv_bias; a.u_out = u_out;
    return mamba::launch_state_update(a) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // extern "C"
