"""Pins for the fp64 oracle: each check ties it to something other than itself.

The pages print no numeric worked example for the scan, so the oracle is pinned by
a hand-derived example (tests/golden/hand_worked.json), library routines
(PyTorch's Conv1d, softplus, SiLU; numpy's convolution), closed forms, and the
invariants the pages state (packed documents behave like separate runs; the
associative operator reproduces the recurrence; the SSD matrix form equals the
recurrence for scalar A; the convolutional mode equals the recurrence for a
time-invariant SSM).  Every check runs on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_custom, make_inputs, pack_documents

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
LN2 = math.log(2.0)
LN3 = math.log(3.0)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _scan_case(case, z=None):
    u = np.array(case["u"], dtype=np.float64)[None, :, None]            # (1, L, 1)
    L = u.shape[1]
    if case["dt"] == "ln2":
        delta = np.full((1, L, 1), LN2)
    else:                                                                 # raw 0 through softplus
        delta = np.zeros((1, L, 1))
    A = np.array(case["A"], dtype=np.float64)
    Bm = np.array(case["B"], dtype=np.float64)[None]
    Cm = np.array(case["C"], dtype=np.float64)[None]
    Dv = np.array(case["D"], dtype=np.float64)
    ds = np.array(case["doc_start"], dtype=np.uint8)[None]
    return oracle.selective_scan(u, delta, A, Bm, Cm, Dv, z, None, case["delta_softplus"], ds)


def _ab(pairs, base=LN2):
    return np.array([a * base + b for a, b in pairs])


# ----------------------------------------------------------------------------
# Hand-derived example
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("idx", [0, 1, 2])
def test_hand_worked_scan(idx):
    case = _golden()["scan_cases"][idx]
    out, final = _scan_case(case)
    np.testing.assert_allclose(out[0, :, 0], _ab(case["expected_out"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(final[0, 0], _ab(case["expected_final_state"]), rtol=1e-14, atol=1e-14)


def test_hand_worked_gate():
    g = _golden()
    case = g["scan_cases"][g["gate_case"]["base_case"]]
    z = np.array([LN3, 0.0, -LN3])[None, :, None]
    out, _ = _scan_case(case, z=z)
    base = _ab(case["expected_out"])
    factor = np.array([a * LN3 for a, _ in g["gate_case"]["gate_factor"]])
    np.testing.assert_allclose(out[0, :, 0], base * factor, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("idx", [0, 1])
def test_hand_worked_conv(idx):
    case = _golden()["conv_cases"][idx]
    x = np.array(case["x"], dtype=np.float64)[None, :, None]
    w = np.array(case["weight"], dtype=np.float64)[None, :]
    b = np.array([case["bias"]])
    ds = np.array(case["doc_start"], dtype=np.uint8)[None]
    u = oracle.causal_conv1d(x, w, b, ds, apply_silu=False)
    np.testing.assert_allclose(u[0, :, 0], case["expected"], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# Library routines
# ----------------------------------------------------------------------------
def test_conv_matches_torch_conv1d():
    """Single document: the S6 section's nn.Conv1d(padding=3, groups=D)[..., :L] then SiLU."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    Bt, L, Dm, W = 2, 37, 5, 4
    x = rng.standard_normal((Bt, L, Dm))
    w = rng.uniform(-0.5, 0.5, (Dm, W))
    b = rng.standard_normal(Dm)
    conv = torch.nn.Conv1d(Dm, Dm, W, padding=W - 1, groups=Dm, dtype=torch.float64)
    with torch.no_grad():
        conv.weight.copy_(torch.from_numpy(w)[:, None, :])
        conv.bias.copy_(torch.from_numpy(b))
        ref = conv(torch.from_numpy(x).transpose(1, 2))[..., :L].transpose(1, 2)
        ref = torch.nn.functional.silu(ref).numpy()
    got = oracle.causal_conv1d(x, w, b, None, apply_silu=True)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_elementwise_match_torch():
    torch = pytest.importorskip("torch")
    v = np.concatenate([np.linspace(-80, 80, 2001), [-700.0, 700.0, 0.0, -1e-8, 1e-8]])
    tv = torch.from_numpy(v)
    np.testing.assert_allclose(oracle.softplus(v), torch.nn.functional.softplus(tv, threshold=1e9).numpy(),
                               rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.silu(v), torch.nn.functional.silu(tv).numpy(), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(oracle.sigmoid(v), torch.sigmoid(tv).numpy(), rtol=1e-15, atol=1e-300)


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]    # exact ties go to even
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(a).view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
def _small(seed, heads=False, docs=4.0, L=24, Dm=6, N=3, Bt=2):
    inp = make_custom(Bt, L, Dm, N, nheads=(3 if heads else 0), dtype="f32", docs=docs, seed=seed)
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    return inp, u


@pytest.mark.parametrize("heads", [False, True])
@pytest.mark.parametrize("docs", [None, 4.0])
def test_recurrence_equals_unrolled_closed_form(heads, docs):
    inp, u = _small(5, heads=heads, docs=docs)
    args = (u, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.delta_bias, True, inp.doc_start)
    out, final = oracle.selective_scan(*args)
    out_bf, final_bf = oracle.brute_force_scan(*args)
    np.testing.assert_allclose(out, out_bf, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(final, final_bf, rtol=1e-12, atol=1e-14)


def test_delta_to_zero_leaves_skip_and_gate():
    """delta_bias = -60: softplus ~ 8.8e-27, so out = D u silu(z)."""
    inp, u = _small(6)
    bias = np.full_like(inp.delta_bias, -60.0)
    out, final = oracle.selective_scan(u, np.zeros_like(inp.delta), inp.A, inp.B, inp.C, inp.D, inp.z,
                                       bias, True, inp.doc_start)
    expect = inp.D[None, None, :] * u * oracle.silu(inp.z)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-20)
    assert np.abs(final).max() < 1e-20


@pytest.mark.parametrize("heads", [False, True])
def test_A_zero_is_segmented_cumsum(heads):
    inp, u = _small(7, heads=heads)
    A0 = np.zeros_like(inp.A)
    out, final = oracle.selective_scan(u, inp.delta, A0, inp.B, inp.C, inp.D, None, inp.delta_bias, True,
                                       inp.doc_start)
    dt = oracle.softplus(inp.delta.astype(np.float64) + inp.delta_bias)
    if heads:
        dt = np.repeat(dt, u.shape[2] // inp.A.shape[0], axis=2)
    seg = oracle.doc_segment_start(inp.doc_start, *u.shape[:2])
    Bt, L, Dm = u.shape
    expect = np.zeros_like(out)
    for b in range(Bt):
        for t in range(L):
            s = slice(seg[b, t], t + 1)
            hsum = np.einsum("s,sd,sn->dn", np.ones(t + 1 - seg[b, t]), dt[b, s] * u[b, s], inp.B[b, s])
            expect[b, t] = hsum @ inp.C[b, t] + inp.D * u[b, t]
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-13)


def test_geometric_closed_form():
    """N=1, B=C=u=1, D=0, constant dt, A=-alpha: h_t = dt (1 - q^{t+1}) / (1 - q), q = e^{-alpha dt}."""
    L, alpha, dt = 300, 0.7, 0.05
    one = np.ones((1, L, 1))
    out, final = oracle.selective_scan(one, np.full((1, L, 1), dt), np.array([[-alpha]]), one, one,
                                       np.zeros(1), None, None, False, None)
    q = math.exp(-alpha * dt)
    t = np.arange(L)
    expect = dt * (1 - q ** (t + 1)) / (1 - q)
    np.testing.assert_allclose(out[0, :, 0], expect, rtol=1e-12)
    assert abs(final[0, 0, 0] - expect[-1]) <= 1e-12 * expect[-1]


def test_softplus_inverse_bias():
    """delta = 0 with delta_bias = log(expm1(v)) gives dt = v (Key Training Tips init)."""
    v = np.array([0.001, 0.01, 0.05, 0.1, 1.0, 5.0])
    bias = np.log(np.expm1(v))
    np.testing.assert_allclose(oracle.softplus(bias), v, rtol=1e-14)
    # and through the scan: with A=0, N=1, B=C=1, D=0 the first output equals dt * u
    u = np.ones((1, 1, v.size))
    out, _ = oracle.selective_scan(u, np.zeros((1, 1, v.size)), np.zeros((v.size, 1)), np.ones((1, 1, 1)),
                                   np.ones((1, 1, 1)), None, None, bias, True, None)
    np.testing.assert_allclose(out[0, 0], v, rtol=1e-14)


def test_single_step():
    rng = np.random.default_rng(9)
    Dm, N = 5, 4
    u = rng.standard_normal((1, 1, Dm))
    delta = rng.standard_normal((1, 1, Dm))
    A = -rng.uniform(0.5, 3, (Dm, N))
    Bm = rng.standard_normal((1, 1, N))
    Cm = rng.standard_normal((1, 1, N))
    Dv = rng.standard_normal(Dm)
    out, final = oracle.selective_scan(u, delta, A, Bm, Cm, Dv, None, None, True, None)
    dt = np.log1p(np.exp(delta[0, 0]))
    h = (dt * u[0, 0])[:, None] * Bm[0, 0][None, :]
    np.testing.assert_allclose(final[0], h, rtol=1e-14)
    np.testing.assert_allclose(out[0, 0], h @ Cm[0, 0] + Dv * u[0, 0], rtol=1e-13)


# ----------------------------------------------------------------------------
# Invariants stated on the pages
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("heads", [False, True])
def test_packed_equals_separate(heads):
    """Packing paragraph: each document starts with fresh conv and recurrent state."""
    inp = make_custom(1, 60, 6, 3, nheads=(2 if heads else 0), dtype="f32", docs=8.0, seed=12)
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    out, final = oracle.selective_scan(u, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.delta_bias, True,
                                       inp.doc_start)
    starts = list(np.flatnonzero(inp.doc_start[0])) + [60]
    assert len(starts) > 3
    for s, e in zip(starts[:-1], starts[1:]):
        sl = slice(s, e)
        u_doc = oracle.causal_conv1d(inp.x[:, sl], inp.conv_w, inp.conv_b, None)
        np.testing.assert_array_equal(u_doc, u[:, sl])
        o_doc, f_doc = oracle.selective_scan(u_doc, inp.delta[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl], inp.D,
                                             inp.z[:, sl], inp.delta_bias, True, None)
        np.testing.assert_array_equal(o_doc, out[:, sl])
    np.testing.assert_array_equal(f_doc, final)


@pytest.mark.parametrize("m", [1, 17, 33])
def test_split_and_carry_equals_whole(m):
    """Contiguous shards joined by the carried state and the last W-1 inputs equal the whole run."""
    inp = make_custom(2, 48, 5, 4, dtype="f32", docs=None, seed=13)
    ds = inp.doc_start.copy()
    ds[1, 40] = 1                                      # a document start after the split
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, ds)
    u_tail = oracle.causal_conv1d(inp.x[:, max(m - 3, 0):], inp.conv_w, inp.conv_b, ds[:, max(m - 3, 0):])
    np.testing.assert_array_equal(u_tail[:, m - max(m - 3, 0):], u[:, m:])
    args = lambda sl: (u[:, sl], inp.delta[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl], inp.D, inp.z[:, sl],
                       inp.delta_bias, True)
    out, final = oracle.selective_scan(*args(slice(None)), ds)
    o1, f1 = oracle.selective_scan(*args(slice(0, m)), ds[:, :m])
    o2, f2 = oracle.selective_scan(*args(slice(m, None)), ds[:, m:], initial_state=f1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), out)
    np.testing.assert_array_equal(f2, final)


def test_associative_equals_sequential():
    """Hardware-Aware Parallel Scan: (a1,b1)(+)(a2,b2) = (a1 a2, a2 b1 + b2) reproduces h_t."""
    rng = np.random.default_rng(21)
    for n in [1, 2, 7, 64, 100]:
        a = rng.uniform(0.2, 1.0, n)
        a[rng.uniform(size=n) < 0.1] = 0.0            # document starts
        b = rng.standard_normal(n)
        h, seq = 0.0, []
        for t in range(n):
            h = a[t] * h + b[t]
            seq.append(h)
        np.testing.assert_allclose(oracle.associative_scan(a, b), seq, rtol=1e-13, atol=1e-13)


def test_scan_chain_is_associative_scan():
    """The oracle's per-(d, n) chain equals the associative scan of its (A_bar, B_bar x) pairs."""
    inp, u = _small(22, docs=5.0, Bt=1)
    out, final = oracle.selective_scan(u, inp.delta, inp.A, inp.B, inp.C, None, None, inp.delta_bias, True,
                                       inp.doc_start)
    dt = oracle.softplus(inp.delta.astype(np.float64) + inp.delta_bias)[0]
    starts = inp.doc_start[0].astype(bool)
    starts[0] = True
    d, n = 2, 1
    a = np.exp(dt[:, d] * inp.A[d, n])
    a[starts] = 0.0
    b = dt[:, d] * u[0, :, d] * inp.B[0, :, n]
    h = oracle.associative_scan(a, b)
    np.testing.assert_allclose(h[-1], final[0, d, n], rtol=1e-12)


def test_ssd_matrix_form_equals_recurrence():
    """Mamba-2 SSD section: for scalar-A heads, Y = (M o C B^T) V equals the recurrence."""
    inp = make_custom(2, 40, 8, 5, nheads=2, dtype="f32", docs=9.0, seed=23)
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    args = (u, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.delta_bias, True, inp.doc_start)
    out, _ = oracle.selective_scan(*args)
    np.testing.assert_allclose(oracle.ssd_matrix_scan(*args), out, rtol=1e-11, atol=1e-13)


def test_time_invariant_equals_convolution_mode():
    """Dual Computation Modes: constant dt, B, C gives y = K * u with K_k = C A_bar^k B_bar."""
    rng = np.random.default_rng(24)
    L, N, dt = 50, 4, 0.3
    A = -rng.uniform(0.2, 2.0, N)
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    u = rng.standard_normal(L)
    out, _ = oracle.selective_scan(u[None, :, None], np.full((1, L, 1), dt), A[None, :],
                                   np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), np.array([0.4]), None, None,
                                   False, None)
    np.testing.assert_allclose(out[0, :, 0], oracle.conv_kernel_scan(u, dt, A, Bv, Cv, 0.4), rtol=1e-11,
                               atol=1e-12)


def test_heads_mode_equals_per_channel_mode():
    """Scalar A per head is the per-channel diagonal A repeated over the head's channels and states."""
    inp = make_custom(1, 30, 6, 4, nheads=3, dtype="f32", docs=8.0, seed=25)
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    out_h, fin_h = oracle.selective_scan(u, inp.delta, inp.A, inp.B, inp.C, inp.D, inp.z, inp.delta_bias, True,
                                         inp.doc_start)
    P = 2
    A_ch = np.repeat(inp.A, P)[:, None].repeat(4, axis=1)
    delta_ch = np.repeat(inp.delta, P, axis=2)
    bias_ch = np.repeat(inp.delta_bias, P)
    out_d, fin_d = oracle.selective_scan(u, delta_ch, A_ch, inp.B, inp.C, inp.D, inp.z, bias_ch, True,
                                         inp.doc_start)
    np.testing.assert_array_equal(out_h, out_d)
    np.testing.assert_array_equal(fin_h, fin_d)


def test_conv_one_hot():
    inp = make_custom(2, 40, 4, 2, dtype="f32", docs=6.0, seed=26)
    e3 = np.zeros((4, 4))
    e3[:, 3] = 1.0
    np.testing.assert_array_equal(oracle.causal_conv1d(inp.x, e3, None, inp.doc_start), oracle.silu(inp.x))
    e0 = np.zeros((4, 4))
    e0[:, 0] = 1.0
    got = oracle.causal_conv1d(inp.x, e0, None, inp.doc_start, apply_silu=False)
    seg = oracle.doc_segment_start(inp.doc_start, 2, 40)
    for b in range(2):
        for t in range(40):
            want = inp.x[b, t - 3] if t - 3 >= seg[b, t] else 0.0
            np.testing.assert_array_equal(got[b, t], want)


# ----------------------------------------------------------------------------
# Input generators
# ----------------------------------------------------------------------------
def test_generator_is_deterministic_and_shaped():
    a = make_inputs("tiny_f32")
    b = make_inputs("tiny_f32")
    for k in ("x", "z", "delta", "delta_bias", "A", "B", "C", "conv_w", "doc_start"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    assert a.x.shape == (1, 64, 16) and a.B.shape == (1, 64, 4) and a.A.shape == (16, 4)
    np.testing.assert_array_equal(a.A, -np.arange(1, 5, dtype=np.float32)[None].repeat(16, 0))
    dt = oracle.softplus(a.delta_bias)
    assert dt.min() >= 0.001 - 1e-6 and dt.max() <= 0.1 + 1e-6
    h = make_inputs("heads_32k", seqlen=512)
    assert h.delta.shape == (2, 512, 24) and h.A.shape == (24,) and h.B.shape == (2, 512, 128)
    assert np.all(h.A <= -1.0 + 1e-6) and np.all(h.A >= -16.0 - 1e-5)
    for v in (h.x, h.z, h.delta, h.B, h.C):
        np.testing.assert_array_equal(v, bf16_round(v))


def test_pack_documents_geometric_mean():
    rng = np.random.default_rng(0)
    flags = pack_documents(rng, 4, 200000, 2048)
    assert np.all(flags[:, 0] == 1)
    lengths = np.diff(np.flatnonzero(flags[0]))
    assert abs(lengths.mean() - 2048) < 0.15 * 2048


# ----------------------------------------------------------------------------
# Gradients: central finite differences of the forward oracle
# ----------------------------------------------------------------------------
def _grad_case(seed, softplus=True, with_z=True, with_D=True, with_bias=True):
    rng = np.random.default_rng(seed)
    Bt, L, Dm, N = 2, 11, 3, 4
    u = rng.normal(size=(Bt, L, Dm))
    delta = rng.normal(0.0, 0.5, size=(Bt, L, Dm)) + (0.0 if softplus else 1.0)
    A = -np.exp(rng.normal(size=(Dm, N)))
    B = rng.normal(size=(Bt, L, N))
    C = rng.normal(size=(Bt, L, N))
    D = rng.normal(size=Dm) if with_D else None
    z = rng.normal(size=(Bt, L, Dm)) if with_z else None
    bias = rng.normal(0.0, 0.3, size=Dm) if with_bias else None
    ds = np.zeros((Bt, L), dtype=np.uint8)
    ds[0, 4] = 1
    ds[1, 1] = 1
    ds[1, 7] = 1
    dout = rng.normal(size=(Bt, L, Dm))
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias, delta_softplus=softplus,
                doc_start=ds), dout


def _loss(args, dout):
    out, _ = oracle.selective_scan(args["u"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                   args["z"], args["delta_bias"], args["delta_softplus"], args["doc_start"])
    return float(np.sum(out * dout))


@pytest.mark.parametrize("flags", [dict(), dict(softplus=False), dict(with_z=False, with_D=False, with_bias=False)],
                         ids=str)
def test_gradients_match_finite_differences(flags):
    args, dout = _grad_case(11, **flags)
    g = oracle.selective_scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"], dout, args["D"],
                                  args["z"], args["delta_bias"], args["delta_softplus"], args["doc_start"])
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias"}
    eps = 1e-6
    for arg, gname in names.items():
        if args[arg] is None:
            assert gname not in g
            continue
        x = args[arg]
        for flat in range(x.size):
            orig = x.flat[flat]
            x.flat[flat] = orig + eps
            lp = _loss(args, dout)
            x.flat[flat] = orig - eps
            lm = _loss(args, dout)
            x.flat[flat] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gname].flat[flat]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (arg, flat, fd, an)


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "no_softplus"])
def test_heads_gradients_match_finite_differences(softplus):
    """Scalar-A heads (A (H,), delta (B, L, H), delta_bias (H,)): every input,
    a carried state and a gradient at the final state included, against central
    differences of the heads-mode forward; row 0 continues the carried state,
    row 1 starts a document at token 0 (its d_initial_state is then 0)."""
    rng = np.random.default_rng(31)
    Bt, L, H, P, N = 2, 10, 2, 2, 3
    Dm = H * P
    args = dict(u=rng.normal(size=(Bt, L, Dm)),
                delta=rng.normal(0.0, 0.5, size=(Bt, L, H)) + (0.0 if softplus else 1.0),
                A=-np.exp(rng.normal(size=H)), B=rng.normal(size=(Bt, L, N)), C=rng.normal(size=(Bt, L, N)),
                D=rng.normal(size=Dm), z=rng.normal(size=(Bt, L, Dm)), delta_bias=rng.normal(0.0, 0.3, size=H),
                initial_state=rng.normal(size=(Bt, Dm, N)))
    ds = np.zeros((Bt, L), dtype=np.uint8)
    ds[0, 6] = 1
    ds[1, 0] = 1
    ds[1, 3] = 1
    dout = rng.normal(size=(Bt, L, Dm))
    dfin = rng.normal(size=(Bt, Dm, N))
    g = oracle.selective_scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"], dout, args["D"],
                                  args["z"], args["delta_bias"], softplus, ds, initial_state=args["initial_state"],
                                  d_final_state=dfin)
    assert g["dA"].shape == (H,) and g["ddelta"].shape == (Bt, L, H) and g["ddelta_bias"].shape == (H,)

    def loss():
        out, fin = oracle.selective_scan(args["u"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                         args["z"], args["delta_bias"], softplus, ds,
                                         initial_state=args["initial_state"])
        return float(np.sum(out * dout) + np.sum(fin * dfin))

    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias", "initial_state": "d_initial_state"}
    eps = 1e-6
    for arg, gname in names.items():
        x = args[arg]
        for flat in range(x.size):
            orig = x.flat[flat]
            x.flat[flat] = orig + eps
            lp = loss()
            x.flat[flat] = orig - eps
            lm = loss()
            x.flat[flat] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gname].flat[flat]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (arg, flat, fd, an)
    assert np.all(g["d_initial_state"][1] == 0.0)


@pytest.mark.parametrize("silu_on,docs", [(True, True), (False, True), (True, False)], ids=str)
def test_conv_gradients_match_finite_differences(silu_on, docs):
    """oracle.causal_conv1d_bwd against central differences of oracle.causal_conv1d:
    every element of x, the weights and the bias, in rows with document starts at
    and inside the first taps (so the zeroed taps are exercised)."""
    rng = np.random.default_rng(12)
    Bt, L, Dm, W = 2, 11, 3, 4
    x = rng.standard_normal((Bt, L, Dm))
    w = rng.uniform(-0.7, 0.7, (Dm, W))
    bias = rng.uniform(-0.3, 0.3, Dm)
    ds = np.zeros((Bt, L), dtype=np.uint8)
    if docs:
        ds[0, [2, 3, 7]] = 1
        ds[1, [5, 10]] = 1
    du = rng.standard_normal((Bt, L, Dm))
    dx, dw, db = oracle.causal_conv1d_bwd(x, w, du, bias, ds if docs else None, apply_silu=silu_on)

    def loss():
        return float(np.sum(oracle.causal_conv1d(x, w, bias, ds if docs else None, apply_silu=silu_on) * du))

    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw), (bias, db)):
        for flat in range(arr.size):
            orig = arr.flat[flat]
            arr.flat[flat] = orig + eps
            lp = loss()
            arr.flat[flat] = orig - eps
            lm = loss()
            arr.flat[flat] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.flat[flat]) <= 1e-6 * max(1.0, abs(fd)), (flat, fd, grad.flat[flat])


def test_gradients_with_carried_state_match_finite_differences():
    """With an initial state and a gradient arriving at the final state, the loss is
    sum(dout * out) + sum(d_final * final_state); every input, the initial state
    included, against central differences.  Row 0 continues the carried state at
    token 0, row 1 starts a document there (its d_initial_state is then 0)."""
    args, dout = _grad_case(21)
    rng = np.random.default_rng(22)
    Bt, L, Dm = args["u"].shape
    N = args["B"].shape[-1]
    args["doc_start"][1, 0] = 1
    init = rng.normal(size=(Bt, Dm, N))
    dfin = rng.normal(size=(Bt, Dm, N))
    g = oracle.selective_scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"], dout, args["D"],
                                  args["z"], args["delta_bias"], args["delta_softplus"], args["doc_start"],
                                  initial_state=init, d_final_state=dfin)

    def loss():
        out, fin = oracle.selective_scan(args["u"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                         args["z"], args["delta_bias"], args["delta_softplus"], args["doc_start"],
                                         initial_state=init)
        return float(np.sum(out * dout) + np.sum(fin * dfin))

    assert np.all(g["d_initial_state"][1] == 0.0)
    eps = 1e-6
    pairs = [(args[k], g[v]) for k, v in (("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"),
                                           ("C", "dC"), ("D", "dD"), ("z", "dz"), ("delta_bias", "ddelta_bias"))]
    pairs.append((init, g["d_initial_state"]))
    for x, gx in pairs:
        for flat in range(x.size):
            orig = x.flat[flat]
            x.flat[flat] = orig + eps
            lp = loss()
            x.flat[flat] = orig - eps
            lm = loss()
            x.flat[flat] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gx.flat[flat]) <= 1e-6 * max(1.0, abs(fd)), (flat, fd, gx.flat[flat])


def _conv_with_history(x, hist, w, bias, ds, silu_on):
    """The conv with W-1 tokens of history before token 0, written as its own loop:
    tap j of token t reads x[t - j] (or the history for t - j < 0) unless a
    document starts in (t - j, t]; token 0 starts one only where ds flags it."""
    Bt, L, Dm = x.shape
    W = w.shape[1]
    u = np.zeros((Bt, L, Dm))
    for b in range(Bt):
        for t in range(L):
            acc = bias.copy()
            for j in range(W):
                src = t - j
                if any(ds[b, s] for s in range(max(src + 1, 0), t + 1)):
                    break
                val = x[b, src] if src >= 0 else hist[b, :, W - 1 + src]
                acc = acc + w[:, W - 1 - j] * val
            u[b, t] = acc / (1.0 + np.exp(-acc)) if silu_on else acc
    return u


@pytest.mark.parametrize("silu_on", [True, False])
def test_conv_gradients_with_history_match_finite_differences(silu_on):
    """oracle.causal_conv1d_bwd with conv_state against central differences of a
    direct loop over the taps (history, weights, bias and x); row 1 flags a start
    at token 2, so its taps into the history stop there."""
    rng = np.random.default_rng(23)
    Bt, L, Dm, W = 2, 7, 3, 4
    x = rng.standard_normal((Bt, L, Dm))
    hist = rng.standard_normal((Bt, Dm, W - 1))
    w = rng.uniform(-0.7, 0.7, (Dm, W))
    bias = rng.uniform(-0.3, 0.3, Dm)
    ds = np.zeros((Bt, L), dtype=np.uint8)
    ds[1, 2] = 1
    du = rng.standard_normal((Bt, L, Dm))
    dx, dw, db, dhist = oracle.causal_conv1d_bwd(x, w, du, bias, ds, apply_silu=silu_on, conv_state=hist)
    assert np.allclose(_conv_with_history(x, np.zeros_like(hist), w, bias, np.where(np.arange(L) == 0, 1, ds), silu_on),
                       oracle.causal_conv1d(x, w, bias, ds, apply_silu=silu_on))

    def loss():
        return float(np.sum(_conv_with_history(x, hist, w, bias, ds, silu_on) * du))

    eps = 1e-6
    for arr, grad in ((x, dx), (hist, dhist), (w, dw), (bias, db)):
        for flat in range(arr.size):
            orig = arr.flat[flat]
            arr.flat[flat] = orig + eps
            lp = loss()
            arr.flat[flat] = orig - eps
            lm = loss()
            arr.flat[flat] = orig
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.flat[flat]) <= 1e-6 * max(1.0, abs(fd)), (flat, fd, grad.flat[flat])


def test_backward_of_a_split_row_equals_the_whole_row():
    """A row cut at token 6: the second half's backward with the first half's final
    state carried in gives d_initial_state, which the first half's backward takes
    as d_final_state; the conv's d_conv_state adds to the first half's dx of its
    last 3 tokens.  Every gradient then equals the whole row's."""
    args, dout = _grad_case(24)
    cut = 6
    sl1, sl2 = slice(0, cut), slice(cut, None)
    whole = oracle.selective_scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"], dout, args["D"],
                                      args["z"], args["delta_bias"], args["delta_softplus"], args["doc_start"])
    part = {k: (args[k][:, sl1], args[k][:, sl2]) for k in ("u", "delta", "B", "C", "z", "doc_start")}
    _, fin1 = oracle.selective_scan(part["u"][0], part["delta"][0], args["A"], part["B"][0], part["C"][0], args["D"],
                                    part["z"][0], args["delta_bias"], args["delta_softplus"], part["doc_start"][0])
    g2 = oracle.selective_scan_bwd(part["u"][1], part["delta"][1], args["A"], part["B"][1], part["C"][1],
                                   dout[:, sl2], args["D"], part["z"][1], args["delta_bias"], args["delta_softplus"],
                                   part["doc_start"][1], initial_state=fin1)
    g1 = oracle.selective_scan_bwd(part["u"][0], part["delta"][0], args["A"], part["B"][0], part["C"][0],
                                   dout[:, sl1], args["D"], part["z"][0], args["delta_bias"], args["delta_softplus"],
                                   part["doc_start"][0], d_final_state=g2["d_initial_state"])
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        assert np.allclose(np.concatenate([g1[k], g2[k]], axis=1), whole[k], rtol=1e-12, atol=1e-12), k
    for k in ("dA", "dD", "ddelta_bias"):
        assert np.allclose(g1[k] + g2[k], whole[k], rtol=1e-11, atol=1e-12), k

    rng = np.random.default_rng(25)
    x = rng.standard_normal(args["u"].shape)
    w = rng.uniform(-0.7, 0.7, (x.shape[2], 4))
    bias = rng.uniform(-0.3, 0.3, x.shape[2])
    du = rng.standard_normal(x.shape)
    ds = args["doc_start"]
    dx, dw, db = oracle.causal_conv1d_bwd(x, w, du, bias, ds)
    # The history the second half sees: the inputs of tokens cut-3 .. cut-1, with
    # zeros for those before a document start at or before token cut-1 (the
    # whole row's taps do not cross that start).  Row 0 starts one at token 4.
    hist = np.transpose(x[:, cut - 3:cut], (0, 2, 1)).copy()
    live = np.array([[not ds[b, cut - 3 + k + 1:cut].any() for k in range(3)] for b in range(x.shape[0])])
    assert not live.all()
    hist *= live[:, None, :]
    dx1, dw1, db1 = oracle.causal_conv1d_bwd(x[:, sl1], w, du[:, sl1], bias, ds[:, sl1])
    dx2, dw2, db2, dh2 = oracle.causal_conv1d_bwd(x[:, sl2], w, du[:, sl2], bias, ds[:, sl2], conv_state=hist)
    dx1[:, cut - 3:cut] += np.transpose(dh2 * live[:, None, :], (0, 2, 1))
    assert np.allclose(np.concatenate([dx1, dx2], axis=1), dx, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw1 + dw2, dw, rtol=1e-11) and np.allclose(db1 + db2, db, rtol=1e-11)


def test_conv_gradient_of_one_hot_weights():
    """With w = e_3 (the current token only) and no SiLU the conv is the identity:
    dx = du and dw[:, 3] = sum_t du x (closed form), in every document."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 9, 4))
    du = rng.standard_normal((2, 9, 4))
    w = np.zeros((4, 4))
    w[:, 3] = 1.0
    ds = np.zeros((2, 9), dtype=np.uint8)
    ds[0, 4] = 1
    dx, dw, db = oracle.causal_conv1d_bwd(x, w, du, None, ds, apply_silu=False)
    assert np.allclose(dx, du, rtol=0, atol=1e-15)
    assert np.allclose(dw[:, 3], np.einsum("bld,bld->d", du, x), rtol=1e-14, atol=1e-14)
    assert np.allclose(db, du.sum(axis=(0, 1)), rtol=1e-14, atol=1e-14)
