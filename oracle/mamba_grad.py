"""Plain fp64 gradients of the selective scan (reverse mode of the sequential
recurrence) and of the causal conv1d in front of it.

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`: the library never imports
it.  The forward is the one of `mamba_oracle.selective_scan` ("Mamba & State
Space Models (SSMs)" skill page: the S6 block diagram and code, "Core Concept"
for the D term; axolotl "FLA Mamba and Mamba2": per-document restart); the
gradients are that forward's adjoint, written step by step backwards in time.
Per channel d and state n, with a_t = exp(dt_t A[n]) (0 at a document start),
h_t = a_t h_{t-1} + dt_t u_t B_t[n], y_t = C_t . h_t + D u_t, out_t = y_t silu(z_t):

    dy_t    = dout_t silu(z_t),        dz_t = dout_t y_t silu'(z_t)
    g_t     = dL/dh_t = C_t dy_t + a_{t+1} g_{t+1}          (a_L g_L = dL/d(final state), 0 if not given)
    dC_t   += dy_t h_t                (summed over channels)
    dB_t   += g_t dt_t u_t            (summed over channels)
    du_t    = dy_t D + sum_n g_t[n] dt_t B_t[n]
    ddt_t   = sum_n g_t[n] (u_t B_t[n] + A[n] a_t[n] h_{t-1}[n])   (second term 0 at a start)
    dA[n]  += g_t[n] dt_t a_t[n] h_{t-1}[n]
    dD     += dy_t u_t
    ddelta_t = ddt_t softplus'(delta_t + bias) = ddt_t sigmoid(delta_t + bias)
    dbias  += ddelta_t
    dh_{-1} = a_0 g_0                  (the carried-in state, when one is given)

Pinned by central finite differences of `selective_scan` (tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

from .mamba_oracle import _f64, doc_segment_start, sigmoid, silu


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
                       doc_start=None, initial_state=None, d_final_state=None):
    """Gradients of sum(dout * out) + sum(d_final_state * final_state) for the
    selective scan.  ``initial_state`` (B, D, N), if given, is the state before
    token 0 (token 0 then starts a document only where doc_start flags it, as in
    the forward); ``d_final_state`` (B, D, N) is the gradient arriving at the
    state after the last token (zero if None).  Returns a dict with du, ddelta,
    dA, dB, dC and, when the input is given, dD, dz, ddelta_bias,
    d_initial_state (all float64).

    A of shape (D, N): per-channel A, delta (B, L, D), delta_bias (D,).
    A of shape (H,): scalar-A heads ("Mamba-2 (SSD)" section of the skill page),
    delta (B, L, H), delta_bias (H,), channel d in head d // (D / H).  The heads
    form is the per-channel scan whose A (on every state), step size and bias
    are shared by the channels of a head; the gradient of a shared parameter is
    the sum of the gradients of its copies, so dA (H,), ddelta (B, L, H) and
    ddelta_bias (H,) sum the per-channel ones over the head's channels (and dA
    over the states)."""
    Am = _f64(A)
    if Am.ndim == 2:
        return _channels_bwd(u, delta, Am, B, C, dout, D, z, delta_bias, delta_softplus, doc_start, initial_state,
                             d_final_state)
    H = Am.shape[0]
    Dm = np.shape(u)[2]
    N = np.shape(B)[-1]
    head = np.arange(Dm) // (Dm // H)                 # head of each channel
    A_ch = np.repeat(Am[head][:, None], N, axis=1)
    delta_ch = _f64(delta)[:, :, head]
    bias_ch = None if delta_bias is None else _f64(delta_bias)[head]
    g = _channels_bwd(u, delta_ch, A_ch, B, C, dout, D, z, bias_ch, delta_softplus, doc_start, initial_state,
                      d_final_state)
    fold = np.zeros((Dm, H))
    fold[np.arange(Dm), head] = 1.0                   # sums a channel's gradient into its head
    g["dA"] = g["dA"].sum(axis=1) @ fold
    g["ddelta"] = g["ddelta"] @ fold
    if "ddelta_bias" in g:
        g["ddelta_bias"] = g["ddelta_bias"] @ fold
    return g


def _channels_bwd(u, delta, A, B, C, dout, D, z, delta_bias, delta_softplus, doc_start, initial_state,
                  d_final_state):
    """selective_scan_bwd for per-channel A (D, N)."""
    u = _f64(u)
    dl = _f64(delta)
    Am = _f64(A)
    Bm = _f64(B)
    Cm = _f64(C)
    go = _f64(dout)
    Bt, L, Dm = u.shape
    N = Bm.shape[-1]
    bias = np.zeros(Dm) if delta_bias is None else _f64(delta_bias)
    pre = dl + bias[None, None, :]
    dt = np.log1p(np.exp(-np.abs(pre))) + np.maximum(pre, 0.0) if delta_softplus else pre
    Dv = np.zeros(Dm) if D is None else _f64(D)
    zz = None if z is None else _f64(z)
    first_is_start = initial_state is None
    starts = doc_segment_start(doc_start, Bt, L, first_is_start=first_is_start) == np.arange(L)[None, :]
    h_init = np.zeros((Bt, Dm, N)) if initial_state is None else _f64(initial_state)

    # Forward, keeping every state and decay (the oracle can afford it).
    a = np.empty((Bt, L, Dm, N))
    h = np.empty((Bt, L, Dm, N))
    hprev = h_init.copy()
    for t in range(L):
        at = np.exp(dt[:, t, :, None] * Am[None, :, :])
        at[starts[:, t]] = 0.0
        a[:, t] = at
        hprev = at * hprev + (dt[:, t, :] * u[:, t, :])[:, :, None] * Bm[:, t, None, :]
        h[:, t] = hprev
    y = np.einsum("bldn,bln->bld", h, Cm) + Dv[None, None, :] * u

    if zz is not None:
        sg = sigmoid(zz)
        dy = go * silu(zz)
        dz = go * y * sg * (1.0 + zz * (1.0 - sg))
    else:
        dy = go
        dz = None

    du = dy * Dv[None, None, :]
    ddt = np.zeros((Bt, L, Dm))
    dA = np.zeros((Dm, N))
    dB = np.zeros((Bt, L, N))
    dC = np.einsum("bld,bldn->bln", dy, h)
    g = np.zeros((Bt, Dm, N))
    for t in range(L - 1, -1, -1):
        if t + 1 < L:
            g = a[:, t + 1] * g
        else:
            g = np.zeros((Bt, Dm, N)) if d_final_state is None else _f64(d_final_state).copy()
        g = g + Cm[:, t, None, :] * dy[:, t, :, None]
        h_before = h[:, t - 1] if t > 0 else h_init
        q = a[:, t] * h_before                                     # 0 at a start
        dB[:, t] = np.einsum("bdn,bd->bn", g, dt[:, t] * u[:, t])
        du[:, t] += np.einsum("bdn,bn->bd", g, Bm[:, t]) * dt[:, t]
        ddt[:, t] = np.einsum("bdn,bn->bd", g, Bm[:, t]) * u[:, t] + np.einsum("bdn,dn->bd", g * q, Am)
        dA += np.einsum("bdn,bd->dn", g * q, dt[:, t])

    ddelta = ddt * sigmoid(pre) if delta_softplus else ddt
    grads = {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC}
    if D is not None:
        grads["dD"] = np.einsum("bld,bld->d", dy, u)
    if zz is not None:
        grads["dz"] = dz
    if delta_bias is not None:
        grads["ddelta_bias"] = ddelta.sum(axis=(0, 1))
    if initial_state is not None:
        grads["d_initial_state"] = (a[:, 0] * g) if L > 0 else (
            np.zeros((Bt, Dm, N)) if d_final_state is None else _f64(d_final_state).copy())
    return grads


def causal_conv1d_bwd(x, weight, du, bias=None, doc_start=None, apply_silu=True, conv_state=None):
    """Gradients of sum(du * u) for u = causal_conv1d(x, weight, bias, doc_start,
    apply_silu) ([S] S6 code: Conv1d with left padding W-1, first L outputs, SiLU;
    [A] packing: taps before the token's document start are zero).  With
    acc_t = bias + sum_j w[W-1-j] x_{t-j} over the taps inside t's document and
    dacc_t = du_t silu'(acc_t) (du_t without SiLU):
        dx_s      = sum_j dacc_{s+j} w[W-1-j]   over the j with s inside (s+j)'s document
        dw[W-1-j] = sum_t dacc_t x_{t-j}        over the same taps
        dbias     = sum_t dacc_t
    Returns dx (B, L, D), dweight (D, W) and dbias (D,), float64.

    ``conv_state`` (B, D, W-1), if given, holds the inputs of the W-1 tokens
    before token 0 (oldest first), and token 0 then starts a document only where
    doc_start flags it.  Those tokens are differentiated as a prefix of the row
    whose own outputs are not part of the loss, and the result gains a fourth
    entry, their gradient d_conv_state (B, D, W-1)."""
    if conv_state is not None:
        hist = np.transpose(_f64(conv_state), (0, 2, 1))            # (B, W-1, D)
        Bt, L, Dm = np.shape(x)
        k = hist.shape[1]
        flags = np.zeros((Bt, L), dtype=np.uint8) if doc_start is None else (np.asarray(doc_start) != 0)
        ds_ext = np.concatenate([np.zeros((Bt, k), dtype=np.uint8), flags.astype(np.uint8)], axis=1)
        ds_ext[:, 0] = 1                                            # the prefix's own start
        dx_ext, dw, db = causal_conv1d_bwd(np.concatenate([hist, _f64(x)], axis=1), weight,
                                           np.concatenate([np.zeros((Bt, k, Dm)), _f64(du)], axis=1),
                                           bias, ds_ext, apply_silu)
        return dx_ext[:, k:], dw, db, np.transpose(dx_ext[:, :k], (0, 2, 1))
    x = _f64(x)
    w = _f64(weight)
    g = _f64(du)
    Bt, L, Dm = x.shape
    W = w.shape[1]
    seg = doc_segment_start(doc_start, Bt, L)
    t = np.arange(L)
    acc = np.zeros((Bt, L, Dm))
    if bias is not None:
        acc += _f64(bias)[None, None, :]
    taps = []
    for j in range(W):
        xs = np.zeros_like(x)
        xs[:, j:, :] = x[:, :L - j, :]
        valid = ((t - j)[None, :] >= seg)[..., None]      # tap j of token t is inside its document
        taps.append((xs, valid))
        acc += np.where(valid, xs, 0.0) * w[:, W - 1 - j][None, None, :]
    if apply_silu:
        sg = sigmoid(acc)
        dacc = g * sg * (1.0 + acc * (1.0 - sg))
    else:
        dacc = g
    dx = np.zeros_like(x)
    dw = np.zeros((Dm, W))
    for j, (xs, valid) in enumerate(taps):
        contrib = np.where(valid, dacc, 0.0)                # d acc_t / d x_{t-j} = w[W-1-j] on valid taps
        dx[:, :L - j, :] += contrib[:, j:, :] * w[:, W - 1 - j][None, None, :]
        dw[:, W - 1 - j] = np.einsum("bld,bld->d", contrib, xs)
    return dx, dw, dacc.sum(axis=(0, 1))
