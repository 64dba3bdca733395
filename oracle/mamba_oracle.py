"""Plain fp64 reference for the Mamba selective-scan forward path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Everything is computed in
float64 with numpy, step by step in the order the pages state it, with no
blocking, fusion or reordering.

Sources (page title, then section):

* "Mamba & State Space Models (SSMs)" skill page (ml-skills):
  - "Core Concept: State Space Models": y = C h + D x (the D skip term);
  - "Discretization" and the S6 block diagram ("Inside one Mamba-1 (S6)
    block"): A_bar_t = exp(delta_t A), B_bar_t = delta_t B_t,
    h_t = A_bar_t * h_{t-1} + B_bar_t x_t, y_t = C_t h_t;
  - "Mamba: Selective State Spaces (S6)": depthwise Conv1d with
    padding = d_conv - 1 keeping the first L outputs, SiLU after the conv,
    dt = softplus(dt), selective_scan(x, dt, A, B, C, D), y * silu(z);
  - "Hardware-Aware Parallel Scan": the associative operator
    (a1, b1) (+) (a2, b2) = (a1 a2, a2 b1 + b2);
  - "Mamba-2: Structured State Space Duality (SSD)": for scalar-times-identity
    A the scan equals Y = (M o (C B^T)) V with M the cumulative products of A;
  - "Dual Computation Modes": for a time-invariant SSM the recurrence equals a
    convolution with K = (C B_bar, C A_bar B_bar, C A_bar^2 B_bar, ...);
  - "Key Training Tips": dt bias is the inverse softplus of its target range.
* axolotl "FLA Mamba and Mamba2" page: in packed rows the convolution and the
  recurrent state start independently for each document.

Readings of points the pages leave open (each is also listed in the design
notes): B_bar = delta * B (not the ZOH form); A is diagonal per channel (or
one scalar per head in the Mamba-2 shape) and is passed already negative; delta
is per channel (per head in the Mamba-2 shape) and delta_bias is added before
the softplus; a document start zeroes both the recurrent state and the
convolution history, and token 0 always starts a document; final_state is the
state after the last token of the row.

All functions are pinned by tests against closed forms, invariants, library
routines and a hand-worked example; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Document structure (axolotl page, packing paragraph)
# ----------------------------------------------------------------------------
def doc_segment_start(doc_start, batch, seqlen, first_is_start=True):
    """seg[b, t] = index of the first token of the document that holds token t.

    ``doc_start`` is (B, L) with nonzero at document starts, or None for one
    document per row.  With ``first_is_start`` token 0 always starts a document;
    otherwise a row whose token 0 is not flagged continues a document begun
    before the row, and those tokens get a very negative seg."""
    if doc_start is None:
        start = np.zeros((batch, seqlen), dtype=bool)
    else:
        start = (np.asarray(doc_start) != 0).copy()
    if seqlen == 0:
        return np.zeros((batch, 0), dtype=np.int64)
    if first_is_start:
        start[:, 0] = True
    before_row = np.int64(-(1 << 62))
    idx = np.where(start, np.arange(seqlen, dtype=np.int64)[None, :], before_row)
    return np.maximum.accumulate(idx, axis=1)


# ----------------------------------------------------------------------------
# Elementwise functions
# ----------------------------------------------------------------------------
def softplus(v):
    """log(1 + e^v), evaluated without overflow: max(v, 0) + log1p(e^-|v|)."""
    v = _f64(v)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def sigmoid(v):
    """1 / (1 + e^-v), evaluated without overflow."""
    v = _f64(v)
    e = np.exp(-np.abs(v))
    return np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(v):
    """SiLU(v) = v * sigmoid(v)."""
    v = _f64(v)
    return v * sigmoid(v)


# ----------------------------------------------------------------------------
# Depthwise causal conv1d (S6 section: each channel filtered on its own, three
# zero taps of left padding, first L outputs kept, then SiLU)
# ----------------------------------------------------------------------------
def causal_conv1d(x, weight, bias=None, doc_start=None, apply_silu=True):
    """u[b,t,d] = act(bias[d] + sum_j weight[d, W-1-j] * x[b, t-j, d]).

    PyTorch's Conv1d is a cross-correlation; with left zero padding of W-1 and the
    first L outputs kept, weight[:, W-1] multiplies the current token and
    weight[:, W-1-j] the token j steps back.  A tap whose token lies before the
    start of token t's document (or before the row) contributes zero."""
    x = _f64(x)
    w = _f64(weight)
    Bt, L, Dm = x.shape
    W = w.shape[1]
    seg = doc_segment_start(doc_start, Bt, L)
    acc = np.zeros((Bt, L, Dm))
    if bias is not None:
        acc += _f64(bias)[None, None, :]
    t = np.arange(L)
    for j in range(W):
        src = t - j                                   # token index of this tap
        xs = np.zeros_like(x)                         # xs[:, t] = x[:, t - j] (zero before the row)
        xs[:, j:, :] = x[:, :L - j, :]
        valid = src[None, :] >= seg                   # tap inside token t's document
        acc += np.where(valid[..., None], xs, 0.0) * w[:, W - 1 - j][None, None, :]
    return silu(acc) if apply_silu else acc


# ----------------------------------------------------------------------------
# Selective scan, sequential recurrence (S6 block diagram + Core Concept)
# ----------------------------------------------------------------------------
def _step_sizes(delta, delta_bias, delta_softplus):
    dt = _f64(delta)
    if delta_bias is not None:
        dt = dt + _f64(delta_bias)[None, None, :]
    return softplus(dt) if delta_softplus else dt


def _channel_params(A, dt, Dm):
    """Per-channel A (D, N) and step sizes (B, L, D) for either A layout."""
    A = _f64(A)
    if A.ndim == 1:                                   # one scalar A per head
        H = A.shape[0]
        assert Dm % H == 0, "dim must be a multiple of the head count"
        P = Dm // H
        return np.repeat(A, P), np.repeat(dt, P, axis=2), True
    return A, dt, False


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                   doc_start=None, initial_state=None):
    """Sequential selective scan.  Returns (out (B,L,D), final_state (B,D,N)).

    Per channel d and state n, for t = 0 .. L-1:
        if t starts a document: h <- 0
        dt_t = softplus(delta[t] + delta_bias)            (or without softplus)
        h <- exp(dt_t * A[d, n]) * h + dt_t * u[t, d] * B[t, n]
        y_t = sum_n C[t, n] h[n] + D[d] u[t, d]
        out_t = y_t * silu(z[t, d])                          (if z is given)
    With ``A`` of shape (H,) (Mamba-2 shape) channel d belongs to head d // P,
    uses A[head] for every state and the head's step size.

    ``initial_state`` (B, D, N), if given, is the state before token 0, and token 0
    then resets only where ``doc_start[b, 0]`` is set."""
    u = _f64(u)
    Bm = _f64(B)
    Cm = _f64(C)
    Bt, L, Dm = u.shape
    N = Bm.shape[-1]
    dt = _step_sizes(delta, delta_bias, delta_softplus)
    A_ch, dt_ch, heads = _channel_params(A, dt, Dm)
    Dv = np.zeros(Dm) if D is None else _f64(D)
    zz = None if z is None else _f64(z)
    if initial_state is None:
        h = np.zeros((Bt, Dm, N))
        seg = doc_segment_start(doc_start, Bt, L, first_is_start=True)
    else:
        h = _f64(initial_state).copy()
        seg = doc_segment_start(doc_start, Bt, L, first_is_start=False)
    starts = seg == np.arange(L)[None, :]             # (B, L) token t starts a document
    out = np.empty((Bt, L, Dm))
    for t in range(L):
        h[starts[:, t]] = 0.0
        d_t = dt_ch[:, t, :]                                     # (B, D)
        if heads:
            a = np.exp(d_t * A_ch[None, :])[:, :, None]          # same decay for every state
        else:
            a = np.exp(d_t[:, :, None] * A_ch[None, :, :])       # (B, D, N)
        bx = (d_t * u[:, t, :])[:, :, None] * Bm[:, t, None, :]  # B_bar * x
        h = a * h + bx
        y = np.einsum("bdn,bn->bd", h, Cm[:, t, :]) + Dv[None, :] * u[:, t, :]
        if zz is not None:
            y = y * silu(zz[:, t, :])
        out[:, t, :] = y
    return out, h


# ----------------------------------------------------------------------------
# Unrolled closed form: y_t = sum_{s in doc(t), s <= t} C_t (prod_{s<r<=t} A_bar_r) B_bar_s x_s
# ----------------------------------------------------------------------------
def brute_force_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                     doc_start=None):
    """O(L^2 D N) unrolled form of the recurrence, for tiny inputs only.

    Each decay product is formed factor by factor from the individual
    exp(dt_r A) values, so it checks the recurrence's indexing independently."""
    u = _f64(u)
    Bm = _f64(B)
    Cm = _f64(C)
    Bt, L, Dm = u.shape
    N = Bm.shape[-1]
    dt = _step_sizes(delta, delta_bias, delta_softplus)
    A_ch, dt_ch, heads = _channel_params(A, dt, Dm)
    A_full = np.repeat(A_ch[:, None], N, axis=1) if heads else A_ch          # (D, N)
    Dv = np.zeros(Dm) if D is None else _f64(D)
    seg = doc_segment_start(doc_start, Bt, L)
    out = np.zeros((Bt, L, Dm))
    final = np.zeros((Bt, Dm, N))
    for b in range(Bt):
        abar = np.exp(dt_ch[b][:, :, None] * A_full[None, :, :])             # (L, D, N)
        bbar = dt_ch[b][:, :, None] * Bm[b][:, None, :]                       # (L, D, N)
        for t in range(L):
            h_t = np.zeros((Dm, N))
            for s in range(seg[b, t], t + 1):
                prod = np.ones((Dm, N))
                for r in range(s + 1, t + 1):
                    prod = prod * abar[r]
                h_t = h_t + prod * bbar[s] * u[b, s][:, None]
            y = h_t @ Cm[b, t] + Dv * u[b, t]
            if z is not None:
                y = y * silu(_f64(z)[b, t])
            out[b, t] = y
            if t == L - 1:
                final[b] = h_t
    return out, final


# ----------------------------------------------------------------------------
# SSD matrix form for scalar-A heads (Mamba-2 SSD section)
# ----------------------------------------------------------------------------
def ssd_matrix_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                    doc_start=None):
    """Attention-like form Y = (M o C B^T) V for A of shape (H,).

    For head h, M[t, s] = exp(A_h (S_t - S_s)) for s <= t in the same document
    (S = cumulative sum of the head's step sizes), else 0; V = dt * x.  This is the
    product of the decays A_bar_r for s < r <= t written as one exponential."""
    u = _f64(u)
    Bm = _f64(B)
    Cm = _f64(C)
    A = _f64(A)
    assert A.ndim == 1, "the SSD form needs one scalar A per head"
    Bt, L, Dm = u.shape
    H = A.shape[0]
    P = Dm // H
    dt = _step_sizes(delta, delta_bias, delta_softplus)          # (B, L, H)
    Dv = np.zeros(Dm) if D is None else _f64(D)
    seg = doc_segment_start(doc_start, Bt, L)
    out = np.zeros((Bt, L, Dm))
    t_idx = np.arange(L)
    for b in range(Bt):
        same_doc = (seg[b][:, None] == seg[b][None, :]) & (t_idx[None, :] <= t_idx[:, None])
        G = Cm[b] @ Bm[b].T                                       # (L, L): C_t . B_s
        for h in range(H):
            S = np.cumsum(dt[b, :, h])
            M = np.where(same_doc, np.exp(A[h] * (S[:, None] - S[None, :])), 0.0)
            V = dt[b, :, h][:, None] * u[b, :, h * P:(h + 1) * P]  # (L, P)
            out[b, :, h * P:(h + 1) * P] = (M * G) @ V
    out = out + Dv[None, None, :] * u
    if z is not None:
        out = out * silu(_f64(z))
    return out


# ----------------------------------------------------------------------------
# Associative (parallel-prefix) form of one scalar recurrence
# ----------------------------------------------------------------------------
def _combine(left, right):
    """(a1, b1) (+) (a2, b2) = (a1 a2, a2 b1 + b2): left is the earlier segment."""
    a1, b1 = left
    a2, b2 = right
    return a1 * a2, a2 * b1 + b2


def associative_scan(a, b):
    """Inclusive scan of pairs (a_t, b_t) with (+), work-efficient tree order.

    Up-sweep builds a reduction tree, down-sweep turns it into exclusive prefixes
    (Blelloch), then each element is combined with its exclusive prefix.  Returns
    the b part, i.e. h_t of h_t = a_t h_{t-1} + b_t from h_{-1} = 0."""
    a = _f64(a).ravel()
    b = _f64(b).ravel()
    n = a.shape[0]
    if n == 0:
        return b.copy()
    size = 1
    while size < n:
        size *= 2
    A_ = np.ones(size)
    B_ = np.zeros(size)
    A_[:n] = a
    B_[:n] = b
    tree_a = A_.copy()
    tree_b = B_.copy()
    step = 1
    while step < size:                                # up-sweep
        for i in range(2 * step - 1, size, 2 * step):
            tree_a[i], tree_b[i] = _combine((tree_a[i - step], tree_b[i - step]),
                                            (tree_a[i], tree_b[i]))
        step *= 2
    tree_a[size - 1], tree_b[size - 1] = 1.0, 0.0     # identity
    step = size // 2
    while step >= 1:                                  # down-sweep
        for i in range(2 * step - 1, size, 2 * step):
            left = (tree_a[i - step], tree_b[i - step])
            parent = (tree_a[i], tree_b[i])
            tree_a[i - step], tree_b[i - step] = parent
            tree_a[i], tree_b[i] = _combine(parent, left)
        step //= 2
    excl_a, excl_b = tree_a[:n], tree_b[:n]
    _, incl_b = _combine((excl_a, excl_b), (a, b))
    return incl_b


# ----------------------------------------------------------------------------
# Convolutional mode for a time-invariant SSM ("Dual Computation Modes")
# ----------------------------------------------------------------------------
def conv_kernel_scan(u, dt, A, Bvec, Cvec, D=0.0):
    """One channel, constant step dt, constant B, C (N,), one document.

    K_k = C . (A_bar^k * B_bar) with A_bar = exp(dt A), B_bar = dt B, and
    y = K * u (causal convolution) + D u."""
    u = _f64(u).ravel()
    A = _f64(A).ravel()
    Bvec = _f64(Bvec).ravel()
    Cvec = _f64(Cvec).ravel()
    L = u.shape[0]
    abar = np.exp(dt * A)
    bbar = dt * Bvec
    K = np.array([np.sum(Cvec * abar ** k * bbar) for k in range(L)])
    return np.convolve(u, K)[:L] + D * u
