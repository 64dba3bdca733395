/*
 * mamba_hip.h -- C ABI of the MI355X (gfx950) Mamba selective-scan path.
 *
 * The two operations of the forward path, each one or more HIP kernel launches on
 * the caller's stream:
 *
 *   mamba_causal_conv1d_fwd   depthwise causal conv1d (width 4) + optional SiLU.
 *       Defined by the "Mamba: Selective State Spaces (S6)" section of the Mamba
 *       skill page (a per-channel causal convolution of width 4: each channel
 *       filtered on its own, three zero taps of left padding, only the first L
 *       outputs kept, then SiLU) and by the packing
 *       paragraph of the axolotl "FLA Mamba and Mamba2" page (the convolution
 *       state starts fresh at every document start).
 *
 *   mamba_selective_scan_fwd  the selective scan with input-dependent
 *       discretisation, D skip and SiLU(z) gate.  Defined by the same skill page:
 *       S6 block diagram (A_bar_t = exp(dt_t A), B_bar_t = dt_t B_t,
 *       h_t = A_bar_t * h_{t-1} + B_bar_t x_t, y_t = C_t h_t), "Core Concept"
 *       (y = C h + D x), the S6 code (dt = softplus(dt), y * silu(z)), the
 *       "Mamba-2 (SSD)" section (scalar A per head, multi-head, headdim), and the
 *       packing paragraph (recurrent state restarts at every document start).
 *
 * Further entry points: the two in one call (mamba_conv_scan_fwd), one-token
 * decode steps, and the backward passes of the conv and of the scan
 * (mamba_causal_conv1d_bwd, mamba_selective_scan_bwd), each described at its
 * declaration below.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees or retains them past the call's completion on the stream.
 *     The library allocates no device memory and keeps no state between calls.
 *   - Layouts are dense row-major: activations (B, L, D) with D contiguous,
 *     B and C (B, L, N), A (D, N) or (H,), final state (B, D, N).
 *   - `dtype` is the storage type of the activations (x, u, delta, B, C, z, out):
 *     MAMBA_DTYPE_F32 or MAMBA_DTYPE_BF16.  Parameters (conv weight/bias, A, D,
 *     delta_bias) and the final state are always float32.  All arithmetic and
 *     the recurrent state are float32; bf16 outputs are rounded to nearest even.
 *   - doc_start is (B, L) uint8; nonzero marks the first token of a document.
 *     Token 0 of every row starts a document, unless the call continues a given
 *     history (conv_state, initial_state: then only where doc_start marks it).
 *     NULL = no starts besides that one.  A document start zeroes the conv
 *     history and the recurrent state.
 *   - `stream` is a hipStream_t (NULL = the null stream).
 *   - Every call validates its arguments before any launch and returns a status
 *     code; no exception crosses the ABI.  Errors raised by a kernel while it
 *     runs surface at the caller's next synchronisation, as for any HIP call.
 *   - Calls are reentrant.  Concurrent calls must not share output or workspace
 *     buffers.  Inputs and outputs must not overlap.
 *   - A call with no tokens (B L D == 0) reads no input and writes only what
 *     has a value without tokens: a final state equal to the initial state (or
 *     0), the adjoint passed through (d_initial_state = d_final_state, or 0),
 *     and zero for the sums over tokens (dA, dD, ddelta_bias, dweight, dbias,
 *     d_conv_state).
 */
#ifndef MAMBA_HIP_H
#define MAMBA_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MAMBA_DTYPE_F32 = 0,
    MAMBA_DTYPE_BF16 = 1
} mamba_dtype_t;

enum {
    MAMBA_OK = 0,
    MAMBA_ERR_INVALID_ARGUMENT = -1, /* null required pointer, bad size, overlap  */
    MAMBA_ERR_UNSUPPORTED = -2,      /* valid but not implemented (width, N, ...) */
    MAMBA_ERR_MISALIGNED = -3,       /* pointer alignment below what is required  */
    MAMBA_ERR_WORKSPACE = -4,        /* workspace missing or too small            */
    MAMBA_ERR_HIP = -5               /* a HIP launch failed                        */
};

/* Library version, (major << 16) | (minor << 8) | patch. */
int mamba_version(void);

/* Static description of a status code (never NULL). */
const char* mamba_status_string(int status);

/* Causal depthwise conv1d.
 *   x         (B, L, D) activations, `dtype`.
 *   weight    (D, width) float32; weight[d, width-1] multiplies the current token,
 *             weight[d, width-1-j] the token j steps back (PyTorch Conv1d layout
 *             with the singleton group dimension dropped).
 *   bias      (D,) float32 or NULL (zero).
 *   doc_start (B, L) uint8 or NULL.
 *   conv_state (B, D, 3) `dtype` or NULL: the inputs x[-3], x[-2], x[-1] before
 *             token 0 of each row (the window mamba_causal_conv1d_update keeps).
 *             With it, token 0 starts a new document only where doc_start[b, 0]
 *             is set; without it, token 0 always does (taps before it read zero).
 *   out       (B, L, D), `dtype`: act(bias + sum_j weight[., width-1-j] x[t-j]),
 *             taps before the start of the token's document read zero;
 *             act = SiLU if apply_silu else identity.
 *   width     must be 4.
 * Alignment: x and out aligned to their element size (16 bytes and D a
 * multiple of 16 bytes' worth of elements select the vectorised kernel).
 * Returns MAMBA_OK, or an error before any launch.  B, L or D of 0 is a no-op. */
int mamba_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                            const uint8_t* doc_start, const void* conv_state, void* out,
                            int64_t batch, int64_t seqlen, int64_t dim, int32_t width,
                            int32_t dtype, int32_t apply_silu, void* stream);

/* Shape of one selective-scan call. */
typedef struct {
    int64_t batch;          /* B                                                   */
    int64_t seqlen;         /* L                                                   */
    int64_t dim;            /* D: channels (d_inner)                               */
    int64_t dstate;         /* N: state size per channel                           */
    int32_t nheads;         /* 0: A is (D, N), delta (B, L, D), delta_bias (D,)    */
                            /* H > 0: A is (H,), delta (B, L, H), delta_bias (H,), */
                            /*        channel d belongs to head d / (D / H)        */
    int32_t ngroups;        /* must be 1: B and C are shared by all channels       */
    int32_t dtype;          /* mamba_dtype_t of u, delta, B, C, z, out             */
    int32_t delta_softplus; /* nonzero: dt = softplus(delta + delta_bias)          */
                            /* zero:    dt = delta + delta_bias                    */
} mamba_scan_dims_t;

/* Bytes of device workspace mamba_selective_scan_fwd needs for `dims`
 * (written to *bytes; may be 0).  Returns a status like the launch itself. */
int mamba_selective_scan_workspace_bytes(const mamba_scan_dims_t* dims, size_t* bytes);

/* Selective scan forward.
 *   u          (B, L, D)         input x_t of the recurrence (the conv output).
 *   delta      (B, L, D|H)       raw step size before bias and softplus.
 *   A          (D, N) | (H,)     float32, the continuous-time decay (pass A < 0,
 *                                e.g. -exp(A_log)); any finite value is accepted.
 *   B, C       (B, L, N)         input and output projections, shared by channels.
 *   D          (D,) float32 or NULL (no skip term).
 *   z          (B, L, D) or NULL (no gate).
 *   delta_bias (D|H,) float32 or NULL (zero).
 *   doc_start  (B, L) uint8 or NULL.
 *   initial_state (B, D, N) float32 or NULL: the state before token 0 of each
 *              row (e.g. the final_state of the preceding stretch of the same
 *              rows).  With it, token 0 starts a new document only where
 *              doc_start[b, 0] is set; without it, token 0 always does and the
 *              state starts at zero.  Must not overlap out, final_state or the
 *              workspace.
 *   out        (B, L, D)         y_t * silu(z_t), y_t = C_t . h_t + D u_t.
 *   final_state (B, D, N) float32 or NULL: h after token L-1 (the state of the
 *                                last document of each row).
 *   workspace  device buffer of at least mamba_selective_scan_workspace_bytes
 *              bytes, 256-byte aligned; contents on entry are ignored, and it is
 *              scratch for chunk carries during the call.  May be NULL when the
 *              required size is 0.
 * Supported (others return MAMBA_ERR_UNSUPPORTED):
 *   ngroups == 1, and (L + 64) * max(D, N) * 4 < 2^31 (a batch row of any
 *   tensor is addressed with 32-bit offsets);
 *   nheads == 0: 1 <= N <= 16;
 *   nheads > 0, float32: 1 <= N <= 128 (recurrent form, fp32 throughout);
 *   nheads > 0, bf16: head size D / H in {32, 64} and 1 <= N <= 128 (chunked
 *   matrix-product form: bf16 operands, fp32 accumulation and state; Mamba
 *   skill page, "Mamba-2: Structured State Space Duality (SSD)").
 *   The kernels are compiled for N = 4, 8, 16 (per channel), 16, 32, 64, 128
 *   (fp32 heads) and multiples of 8 (bf16 heads); any other N runs on copies of
 *   B, C, A and the states padded with zeros to the next such size inside the
 *   workspace (a padded state stays zero and adds nothing: the results are
 *   those of N states).
 * Alignment: activations aligned to their element size; B and C rows must be
 * 4-byte aligned when N is a compiled size (N even for bf16); with nheads > 0
 * and bf16, u, z, out, B and C must be 16-byte aligned (B and C only when N is
 * a multiple of 8).  Otherwise MAMBA_ERR_MISALIGNED.
 * B, L or D of 0 is a no-op.
 * Repeated calls with the same arguments give bitwise identical results. */
int mamba_selective_scan_fwd(const mamba_scan_dims_t* dims,
                             const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D,
                             const void* z, const float* delta_bias,
                             const uint8_t* doc_start, const float* initial_state,
                             void* out, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Selective scan forward that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *   Arguments and results as mamba_selective_scan_fwd without workspace.  The
 *   chunk carries live in a 64 MiB array of the library's own, one per GPU,
 *   held from the library's first use on that GPU until the process ends.  The
 *   step sizes are recomputed in the output pass instead of being handed over
 *   (with bf16 I/O, results may therefore differ from mamba_selective_scan_fwd
 *   by the rounding of dt to bf16, well inside the bf16 tolerance; with fp32 I/O
 *   they are the same).
 *   Carries take 8 (ceil(L / chunk) - 1) B D N bytes (per-channel A, fp32
 *   scalar-A heads; the chunk is 128 to 4096 tokens, chosen so that about 4096
 *   waves run: 50 MB at B = 2, L = 32768, D = 1536, N = 16) or, for bf16
 *   scalar-A heads, the matrix form's segment states (25 MB at B = 2, L = 32768,
 *   24 heads of 64 channels, N = 128).  A call that needs more than 64 MiB
 *   returns MAMBA_ERR_WORKSPACE before any launch.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on
 *   one GPU (different streams or host threads) race and must be serialised by
 *   the caller.  Nothing needs clearing between calls.
 *   MAMBA_ERR_HIP also reports a failed lookup of the array's address. */
int mamba_selective_scan_fwd_noalloc(const mamba_scan_dims_t* dims,
                                     const void* u, const void* delta, const float* A,
                                     const void* B, const void* C, const float* D,
                                     const void* z, const float* delta_bias,
                                     const uint8_t* doc_start, const float* initial_state,
                                     void* out, float* final_state, void* stream);

/* Conv1d (width 4, SiLU) and selective scan in one call: the whole forward path
 * of the mixer core.  Same arguments and results as mamba_causal_conv1d_fwd
 * (x, conv_weight, conv_bias, doc_start, conv_state; apply_silu = 1) followed by
 * mamba_selective_scan_fwd (dims, delta ... final_state, workspace sized by
 * mamba_selective_scan_workspace_bytes) on its output; the conv output is also
 * written to `u` (B, L, D), or not at all when u is NULL (inference needs only
 * out).  With per-channel A the convolution runs inside the scan's first pass,
 * which saves the conv's separate pass over x and u; with u NULL the second pass
 * forms the conv output again from x instead of reading it back.  With bf16
 * scalar-A heads the conv runs first and the scan reads u, or, with u NULL,
 * both passes of the scan form it from x (x then 16-byte aligned, else
 * MAMBA_ERR_MISALIGNED).  fp32 scalar-A heads require u (MAMBA_ERR_UNSUPPORTED
 * for NULL).
 * conv_state and initial_state act on their own stage each, as in the two
 * separate calls: a continuation passes both; a conv_state alone continues
 * the conv's history while the scan's state starts at zero. */
int mamba_conv_scan_fwd(const mamba_scan_dims_t* dims, const void* x, const float* conv_weight,
                        const float* conv_bias, const void* conv_state, const void* delta,
                        const float* A, const void* B, const void* C, const float* D,
                        const void* z, const float* delta_bias, const uint8_t* doc_start,
                        const float* initial_state, void* u, void* out, float* final_state,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---- Backward pass (training) of the conv: the gradients of sum(du * u)
 * through mamba_causal_conv1d_fwd (same pages and sections as the forward).
 * With acc_t = bias + sum_j w[3-j] x_{t-j} over the taps inside token t's
 * document and dacc_t = du_t silu'(acc_t) (du_t when apply_silu == 0):
 *   dx_s = sum_j dacc_{s+j} w[3-j] over the j with s inside (s+j)'s document,
 *   dweight[:, 3-j] = sum_t dacc_t x_{t-j} over the same taps, dbias = sum_t dacc_t.
 * Chained after mamba_selective_scan_bwd (whose du it takes) it completes the
 * mixer core's backward: dx of x, the conv's weight and bias gradients. */

/* Bytes of device workspace mamba_causal_conv1d_bwd needs (per-tile partial
 * sums of the weight gradients: 20 bytes per channel per 48 tokens). */
int mamba_causal_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, size_t* bytes);

/* Conv backward.
 *   x, weight, bias, doc_start, conv_state, apply_silu, width, dtype: as the
 *              forward call (conv_state NULL: token 0 starts a document).
 *   du         (B, L, D)  gradient of the loss with respect to the conv output.
 *   dx         (B, L, D)  written.
 *   dweight    (D, 4) float32, written.
 *   dbias      (D,) float32 or NULL (not computed).
 *   d_conv_state (B, D, 3) float32 or NULL: the gradient with respect to
 *              conv_state (zero where token 0 starts a document); requires
 *              conv_state, else MAMBA_ERR_INVALID_ARGUMENT.  For a row split in
 *              two pieces, the second piece's d_conv_state adds to dx of the
 *              first piece's last three tokens.
 *   workspace  at least mamba_causal_conv1d_bwd_workspace_bytes bytes, 256-byte
 *              aligned, scratch.
 * Outputs must not overlap each other, the inputs or the workspace.  Sums run
 * in a fixed order (repeated calls give identical results). */
int mamba_causal_conv1d_bwd(const void* x, const float* weight, const float* bias, const uint8_t* doc_start,
                            const void* conv_state, const void* du, void* dx, float* dweight, float* dbias,
                            float* d_conv_state, int64_t batch, int64_t seqlen, int64_t dim, int32_t width,
                            int32_t dtype, int32_t apply_silu, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Backward pass (training) of the scan: the gradients of
 * sum(dout * out) through mamba_selective_scan_fwd, i.e. the adjoint of the
 * recurrence run from the row end back to token 0.  Defined by the same pages
 * as the forward; the states are recomputed rather than stored (Mamba skill
 * page, "Hardware-Aware Parallel Scan": recomputation in the backward pass).
 * With a_t = exp(dt_t A) (0 at a document start), h_t the forward state and
 * dy_t = dout_t silu(z_t), the adjoint g_t = C_t dy_t + a_{t+1} g_{t+1} gives
 *   du_t = D dy_t + dt_t (g_t . B_t)
 *   ddelta_t = [u_t (g_t . B_t) + sum_n A g_t a_t h_{t-1}] * sigmoid(delta_t + delta_bias)
 *   dB_t = sum_d g_t dt_t u_t,  dC_t = sum_d dy_t h_t,  dA = sum_t dt_t g_t a_t h_{t-1}
 *   dD = sum_t dy_t u_t,  dz_t = dout_t y_t silu'(z_t),  ddelta_bias = sum_t ddelta_t.
 * With scalar-A heads (nheads > 0; "Mamba-2 (SSD)" section of the Mamba skill
 * page) A, delta and delta_bias are shared by the D / H channels and N states
 * of a head, so their gradients are the sums of the per-channel ones above over
 * those channels and states (dA over all of them, ddelta and ddelta_bias over
 * the head's channels). */

/* Bytes of device workspace mamba_selective_scan_bwd needs for `dims`.
 * Per channel: about B L D (N + 2) * 4 / 16 + B L ceil(D / 128) * 8 N bytes plus
 * the per-chunk carries and two (B, D, N) float32 arrays; 0.68 GB at B = 2,
 * L = 32768, D = 1536, N = 16.  Scalar-A heads: about B D N ceil(L / 16)
 * * 4 (the state entering every 16-token chunk) + 2 B H L N * 4 (per-head dB,
 * dC) bytes; 4.88 GB at B = 2, L = 32768, D = 1536, H = 24, N = 128.  States
 * padded to a compiled size (below) add their zero-padded copies. */
int mamba_selective_scan_bwd_workspace_bytes(const mamba_scan_dims_t* dims, size_t* bytes);

/* Selective scan backward.
 *   dims, u, delta, A, B, C, D, z, delta_bias, doc_start, initial_state: as the
 *              forward call whose gradients are wanted (initial_state NULL:
 *              token 0 starts a document).
 *   dout       (B, L, D)  gradient of the loss with respect to out.
 *   d_final_state (B, D, N) float32 or NULL (= 0): gradient of the loss with
 *              respect to the forward's final_state (the adjoint entering the
 *              row from the right, e.g. from the next piece of a split row).
 *   du, ddelta (B, L, D)  written, dtype `dtype`.
 *   dA         (D, N) float32, written.
 *   dB, dC     (B, L, N)  written, dtype `dtype`.
 *   dD         (D,) float32 or NULL (not computed).  Computed also when D is NULL
 *              (the gradient at D = 0).
 *   dz         (B, L, D); must be non-NULL exactly when z is.
 *   ddelta_bias (D,) float32 or NULL (not computed).
 *   d_initial_state (B, D, N) float32 or NULL (not computed): the gradient with
 *              respect to initial_state, i.e. the adjoint leaving the row at its
 *              start (zero where token 0 starts a document); requires
 *              initial_state, else MAMBA_ERR_INVALID_ARGUMENT.
 *   workspace  at least mamba_selective_scan_bwd_workspace_bytes bytes, 256-byte
 *              aligned, scratch (contents on entry ignored).
 *   With nheads > 0: A, dA (H,); delta, ddelta (B, L, H); delta_bias,
 *              ddelta_bias (H,).
 * Supported: nheads == 0 with 1 <= N <= 16 and, with bf16, an even D; nheads > 0
 * with head size D / H of 32 or 64 and 1 <= N <= 128 (both dtypes; the arithmetic
 * is fp32).  N other than a compiled size (4, 8, 16 per channel; 16, 32, 64, 128
 * for heads) runs on zero-padded copies in the workspace, as the forward.  Also
 * what the forward requires; others return MAMBA_ERR_UNSUPPORTED.  With bf16, u,
 * delta, z and dout must be 4-byte aligned (they are read as pairs of channels),
 * else MAMBA_ERR_MISALIGNED.  Outputs must not overlap each other, the inputs
 * or the workspace.  The sums over channels, tokens and rows run in a fixed
 * order: repeated calls give bitwise identical results. */
int mamba_selective_scan_bwd(const mamba_scan_dims_t* dims, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, const uint8_t* doc_start, const float* initial_state,
                             const void* dout, const float* d_final_state, void* du, void* ddelta, float* dA,
                             void* dB, void* dC, float* dD, void* dz, float* ddelta_bias, float* d_initial_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- One-token decode (Mamba skill page, "Dual Computation Modes": the
 * recurrent mode used for generation).  A prefill with mamba_causal_conv1d_fwd
 * and mamba_selective_scan_fwd followed by these steps gives the same outputs as
 * one long call: the conv window holds the last three inputs x (not u) of each
 * channel, the scan state is final_state. */

/* Causal conv1d for one token per row.
 *   x          (B, D)        input at this token, dtype `dtype`.
 *   conv_state (B, D, 3)     same dtype, in place: (x_{t-3}, x_{t-2}, x_{t-1}) on
 *                            entry, (x_{t-2}, x_{t-1}, x_t) on return (zeros
 *                            before a row's first token).
 *   weight (D, 4), bias (D,) or NULL: as mamba_causal_conv1d_fwd.
 *   reset      (B,) uint8 or NULL: nonzero where the token starts a new document
 *              (the window is cleared first).
 *   out        (B, D)        SiLU(conv) (or the plain conv with apply_silu = 0).
 * Supported: width == 4.  No argument may overlap out. */
int mamba_causal_conv1d_update(const void* x, void* conv_state, const float* weight, const float* bias,
                               const uint8_t* reset, void* out, int64_t batch, int64_t dim, int32_t width,
                               int32_t dtype, int32_t apply_silu, void* stream);

/* Selective-scan recurrence for one token per row.
 *   dims       as mamba_selective_scan_fwd with seqlen == 1.
 *   state      (B, D, N) float32, updated in place (16-byte aligned when N is a
 *              power of two from 4 up, else 4-byte):
 *              h <- exp(dt A) h + dt u B.
 *   u, z, out  (B, D); delta (B, D|H); B, C (B, N); A, D, delta_bias as
 *              mamba_selective_scan_fwd.
 *   reset      (B,) uint8 or NULL: nonzero where the token starts a new document
 *              (the state is zeroed first).
 *   out        = (C . h + D u) silu(z).
 * Supported: 1 <= N <= 128, either A layout, ngroups == 1. */
int mamba_selective_state_update(const mamba_scan_dims_t* dims, float* state, const void* u,
                                 const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const void* z, const float* delta_bias,
                                 const uint8_t* reset, void* out, void* stream);

/* Both decode steps in one launch: mamba_causal_conv1d_update (width 4,
 * apply_silu = 1) followed by mamba_selective_state_update on its output, with
 * identical results (u is rounded to the I/O dtype between the two, as the
 * separate steps store it).
 *   dims, state, delta, A, B, C, D, z, delta_bias, reset, out: as
 *              mamba_selective_state_update.
 *   x          (B, D)     the token's conv input.
 *   conv_state (B, D, 3)  the window, I/O dtype, updated in place.
 *   conv_weight (D, 4), conv_bias (D,) or NULL: float32.
 *   u_out      (B, D) or NULL: the conv output, when the caller wants it.
 * The window and u_out may overlap nothing else of the call. */
int mamba_conv_state_update(const mamba_scan_dims_t* dims, const void* x, void* conv_state, const float* conv_weight,
                            const float* conv_bias, float* state, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* delta_bias,
                            const uint8_t* reset, void* u_out, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_HIP_H */
