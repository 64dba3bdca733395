"""GPU parity of the backward pass of the per-channel selective scan
(mamba_selective_scan_bwd) against the fp64 oracle gradients
(oracle.selective_scan_bwd, itself pinned by finite differences).

Small shapes compare every output element.  At the full workload shapes the
loss gradient dout is nonzero on a few channels only: the adjoint of every other
channel is then exactly zero, so the oracle on those channels alone gives every
output, including dB and dC (sums over all channels), while the GPU still runs
the whole shape."""

import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_cotangent, make_custom, make_inputs

from gpu_helpers import assert_close, to_dev, to_host, torch_mod, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (they fail instead of skipping)")
    import selective_state_space_23_amd as mod
    mod._lib.load()
    return mod


def run_bwd(ssm, dev, u, dout, use_z=True, use_D=True, use_bias=True, softplus=True):
    return ssm.selective_scan_bwd(u, dev["delta"], dev["A"], dev["B"], dev["C"], dout,
                                  D=dev["D"] if use_D else None, z=dev["z"] if use_z else None,
                                  delta_bias=dev["delta_bias"] if use_bias else None, doc_start=dev["doc_start"],
                                  delta_softplus=softplus)


def oracle_bwd(inp, dout, channels=None, use_z=True, use_D=True, use_bias=True, softplus=True):
    ch = np.arange(inp.x.shape[2]) if channels is None else np.asarray(channels)
    return oracle.selective_scan_bwd(inp.x[:, :, ch], inp.delta[:, :, ch], inp.A[ch], inp.B, inp.C,
                                     dout[:, :, ch], D=inp.D[ch] if use_D else None,
                                     z=inp.z[:, :, ch] if use_z else None,
                                     delta_bias=inp.delta_bias[ch] if use_bias else None,
                                     delta_softplus=softplus, doc_start=inp.doc_start)


def compare(got, ref, dtype, what):
    assert set(got) == set(ref), (what, sorted(got), sorted(ref))
    for k in sorted(ref):
        # dA, dD, ddelta_bias are float32 outputs, but their accuracy follows the
        # inputs' precision (bf16 inputs give bf16-level step sizes).
        assert_close(to_host(got[k]), ref[k], dtype, f"{what} {k}")


def bwd_case(ssm, inp, seed, **flags):
    Bt, L, Dm = inp.x.shape
    dout = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=seed)
    dev = upload(inp)
    got = run_bwd(ssm, dev, to_dev(inp.x, inp.dtype), to_dev(dout, inp.dtype), **flags)
    ref = oracle_bwd(inp, dout, **flags)
    compare(got, ref, inp.dtype, f"bwd {inp.x.shape} {inp.dtype} {flags}")


BWD_CASES = [
    # (batch, seqlen, dim, dstate, dtype, docs)
    (1, 64, 16, 4, "f32", None),            # one chunk, one window
    (2, 1000, 100, 16, "bf16", 150.0),      # 8 chunks of 128, a 104-token tail, ragged D
    (2, 777, 64, 8, "bf16", 90.0),
    (1, 500, 70, 4, "f32", 60.0),
    (3, 257, 130, 16, "f32", 40.0),         # the last chunk ends inside a 4-token piece
    (1, 3, 16, 16, "bf16", None),           # fewer tokens than a piece
    (1, 2100, 300, 16, "bf16", 300.0),      # two channel blocks, 17 chunks
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_parity_small(ssm, case):
    Bt, L, Dm, N, dt, docs = case
    inp = make_custom(Bt, L, Dm, N, dtype=dt, docs=docs, seed=800 + L + Dm)
    bwd_case(ssm, inp, seed=900 + L)


@pytest.mark.parametrize("flags", [
    dict(use_z=False), dict(use_D=False), dict(use_bias=False), dict(softplus=False, use_bias=False),
    dict(use_z=False, use_D=False, use_bias=False),
], ids=lambda f: ",".join(f"{k}={v}" for k, v in f.items()))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_optional_inputs(ssm, flags, dtype):
    inp = make_custom(2, 600, 96, 16, dtype=dtype, docs=100.0, seed=811)
    if not flags.get("softplus", True):
        # Without softplus, delta is the step size itself: give positive ones.
        # (Negative steps make exp(dt A) > 1 and the states grow towards 1e36
        # within 600 tokens, where fp32 gradient sums are ill-conditioned.)
        pos = np.abs(inp.delta) * np.float32(0.5) + np.float32(0.001)
        inp.delta[:] = bf16_round(pos) if dtype == "bf16" else pos
    bwd_case(ssm, inp, seed=911, **flags)


def test_bwd_documents_at_block_edges(ssm):
    """Documents starting on chunk, window, 16-token block and piece boundaries,
    one token before and after them, and a one-token document."""
    L = 1200
    inp = make_custom(2, L, 64, 16, dtype="f32", docs=None, seed=812)
    inp.doc_start[:] = 0
    inp.doc_start[:, 0] = 1
    for t in (128, 129, 255, 256, 320, 336, 340, 341, 342, 383, 384, 512, 513, 1023, 1024, 1199):
        inp.doc_start[0, t] = 1
    for t in range(100, L, 97):
        inp.doc_start[1, t] = 1
    bwd_case(ssm, inp, seed=912)


def test_bwd_is_deterministic(ssm):
    torch = torch_mod()
    inp = make_custom(2, 3000, 300, 16, dtype="bf16", docs=400.0, seed=813)
    dout = to_dev(make_cotangent(2, 3000, 300, dtype="bf16", seed=913), "bf16")
    dev = upload(inp)
    u = to_dev(inp.x, "bf16")
    g1 = run_bwd(ssm, dev, u, dout)
    g2 = run_bwd(ssm, dev, u, dout)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


SAMPLES = {"packed_32k": [0, 5, 63, 64, 700, 1535], "m130_2k": [0, 777, 1535], "wide_64k": [0, 1000, 5119]}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_bwd_workload(ssm, name):
    """Full workload shape, dout supported on a few channels: every output is
    compared (zero outside those channels)."""
    torch = torch_mod()
    inp = make_inputs(name)
    Bt, L, Dm = inp.x.shape
    ch = np.array(SAMPLES[name])
    print(f"[bwd] {name} shape={inp.x.shape}", flush=True)
    dout = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=920, channels=ch)
    dev = upload(inp)
    got = run_bwd(ssm, dev, to_dev(inp.x, inp.dtype), to_dev(dout, inp.dtype))
    torch.cuda.synchronize()
    idx = torch.from_numpy(ch).to(got["du"].device)
    others = torch.from_numpy(np.setdiff1d(np.arange(Dm), ch)).to(got["du"].device)
    for k in ("du", "ddelta", "dz"):
        assert torch.count_nonzero(got[k].index_select(2, others)) == 0, f"{name} {k} outside the channels"
    for k in ("dA", "dD", "ddelta_bias"):
        assert torch.count_nonzero(got[k].index_select(0, others)) == 0, f"{name} {k} outside the channels"
    sub = {k: to_host(got[k].index_select(2, idx)) for k in ("du", "ddelta", "dz")}
    sub.update({k: to_host(got[k].index_select(0, idx)) for k in ("dA", "dD", "ddelta_bias")})
    sub.update({k: to_host(got[k]) for k in ("dB", "dC")})
    del dev, got
    ref = oracle_bwd(inp, dout, channels=ch)
    for k in sorted(ref):
        assert_close(sub[k], ref[k], inp.dtype, f"{name} {k}")


# ----------------------------------------------------------------------------
# conv1d backward, alone and chained after the scan backward
# ----------------------------------------------------------------------------
CONV_BWD_CASES = [
    # (batch, seqlen, dim, dtype, docs)
    (2, 200, 64, "bf16", 20.0),       # channel pairs, several 48-token tiles
    (2, 131, 37, "bf16", 9.0),        # odd D: one channel a thread
    (1, 100, 38, "f32", 7.0),         # D = 2 mod 4: f32 channel pairs
    (2, 150, 38, "bf16", 12.0),       # D = 2 mod 4: bf16 channel pairs
    (3, 1, 24, "bf16", None),         # one token
    (2, 3, 24, "bf16", 2.0),          # fewer tokens than the conv width
    (1, 1000, 1536, "bf16", 64.0),
    (2, 500, 64, "f32", None),
]


def conv_bwd_case(ssm, inp, du, silu=True, bias=True, channels=None):
    dev = upload(inp)
    got = ssm.causal_conv1d_bwd(dev["x"], dev["conv_w"], to_dev(du, inp.dtype), dev["conv_b"] if bias else None,
                                dev["doc_start"], apply_silu=silu)
    ch = np.arange(inp.x.shape[2]) if channels is None else np.asarray(channels)
    ref = oracle.causal_conv1d_bwd(inp.x[:, :, ch], inp.conv_w[ch], du[:, :, ch], inp.conv_b[ch] if bias else None,
                                   inp.doc_start, apply_silu=silu)
    idx = torch_mod().from_numpy(ch).to(got[0].device)
    assert_close(to_host(got[0].index_select(2, idx)), ref[0], inp.dtype, "dx")
    assert_close(to_host(got[1].index_select(0, idx)), ref[1], inp.dtype, "dweight")
    if bias:
        assert_close(to_host(got[2].index_select(0, idx)), ref[2], inp.dtype, "dbias")
    else:
        assert got[2] is None


@pytest.mark.parametrize("case", CONV_BWD_CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("silu,bias", [(True, True), (False, False)])
def test_conv_bwd_parity(ssm, case, silu, bias):
    Bt, L, Dm, dt, docs = case
    inp = make_custom(Bt, L, Dm, 4, dtype=dt, docs=docs, seed=830 + L + Dm)
    inp.conv_b[:] = np.linspace(-0.3, 0.3, Dm).astype(np.float32)
    du = make_cotangent(Bt, L, Dm, dtype=dt, seed=930 + L)
    conv_bwd_case(ssm, inp, du, silu, bias)


def test_conv_bwd_documents_at_tile_edges(ssm):
    """Document starts on, one before and one after the 48-token tile edges, and
    within the 3 tokens that a tile reads past its end."""
    L = 300
    inp = make_custom(2, L, 64, 4, dtype="f32", docs=None, seed=831)
    inp.doc_start[:] = 0
    for t in (47, 48, 49, 50, 51, 95, 96, 97, 143, 144, 145, 146, 147, 149, 191, 299):
        inp.doc_start[0, t] = 1
    for t in range(1, L, 3):
        inp.doc_start[1, t] = 1
    du = make_cotangent(2, L, 64, dtype="f32", seed=931)
    conv_bwd_case(ssm, inp, du)


def test_conv_bwd_workload(ssm):
    inp = make_inputs("packed_32k")
    Bt, L, Dm = inp.x.shape
    print(f"[conv bwd] packed_32k shape={inp.x.shape}", flush=True)
    du = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=932)
    conv_bwd_case(ssm, inp, du, channels=[0, 7, 8, 700, 1535])


def test_mixer_core_backward_chain(ssm):
    """conv forward -> scan backward -> conv backward on the GPU against the same
    chain in the oracle: dx, the conv's weight and bias gradients, and the scan's
    parameter gradients of the whole conv + scan forward."""
    inp = make_custom(2, 700, 96, 16, dtype="bf16", docs=120.0, seed=833)
    inp.conv_b[:] = np.linspace(-0.2, 0.2, 96).astype(np.float32)
    Bt, L, Dm = inp.x.shape
    dout = make_cotangent(Bt, L, Dm, dtype="bf16", seed=933)
    dev = upload(inp)
    u = ssm.causal_conv1d_fwd(dev["x"], dev["conv_w"], dev["conv_b"], dev["doc_start"])
    g = ssm.selective_scan_bwd(u, dev["delta"], dev["A"], dev["B"], dev["C"], to_dev(dout, "bf16"), dev["D"],
                               dev["z"], dev["delta_bias"], dev["doc_start"])
    dx, dw, db = ssm.causal_conv1d_bwd(dev["x"], dev["conv_w"], g["du"], dev["conv_b"], dev["doc_start"])
    # oracle: u is stored in bf16 by the forward, which the scan then reads
    u_ref = bf16_round(oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start).astype(np.float32))
    gr = oracle.selective_scan_bwd(u_ref, inp.delta, inp.A, inp.B, inp.C, dout, D=inp.D, z=inp.z,
                                   delta_bias=inp.delta_bias, doc_start=inp.doc_start)
    # and du is stored in bf16 between the two backward calls: the same boundary
    # rounding (the weight gradients sum ~1400 tokens of du and would show it)
    du_r = bf16_round(gr["du"].astype(np.float32))
    dx_r, dw_r, db_r = oracle.causal_conv1d_bwd(inp.x, inp.conv_w, du_r, inp.conv_b, inp.doc_start)
    assert_close(to_host(dx), dx_r, "bf16", "chain dx")
    assert_close(to_host(dw), dw_r, "bf16", "chain dweight")
    assert_close(to_host(db), db_r, "bf16", "chain dbias")
    for k in ("dA", "dB", "dC", "dD", "dz", "ddelta", "ddelta_bias"):
        assert_close(to_host(g[k]), gr[k], "bf16", f"chain {k}")


# ----------------------------------------------------------------------------
# Carried state: a given state before token 0 (initial_state / conv_state) and
# a gradient arriving at the final state (d_final_state)
# ----------------------------------------------------------------------------
CARRY_CASES = [
    # (batch, seqlen, dim, dstate, dtype, docs)
    (2, 64, 16, 4, "f32", None),            # one chunk: no carries between chunks
    (2, 600, 96, 16, "bf16", 100.0),        # several chunks
    (2, 1000, 100, 8, "f32", 300.0),        # ragged D, a 104-token tail
    (2, 3, 16, 16, "bf16", None),           # fewer tokens than a piece
]


def carry_inputs(case, seed):
    Bt, L, Dm, N, dt, docs = case
    inp = make_custom(Bt, L, Dm, N, dtype=dt, docs=docs, seed=seed)
    inp.doc_start[0, 0] = 0       # row 0 continues the given state
    inp.doc_start[1, 0] = 1       # row 1 starts a document at token 0 (its d_initial_state is 0)
    rng = np.random.default_rng(seed + 1)
    init = rng.normal(0.0, 0.5, size=(Bt, Dm, N)).astype(np.float32)
    dfin = rng.normal(0.0, 1.0, size=(Bt, Dm, N)).astype(np.float32)
    return inp, init, dfin


@pytest.mark.parametrize("case", CARRY_CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("with_init,with_dfin", [(True, True), (True, False), (False, True)])
def test_bwd_carried_state(ssm, case, with_init, with_dfin):
    torch = torch_mod()
    inp, init, dfin = carry_inputs(case, seed=840 + case[1] + case[2])
    if not with_init:
        inp.doc_start[:, 0] = 1
    Bt, L, Dm = inp.x.shape
    dout = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=940 + L)
    dev = upload(inp)
    got = ssm.selective_scan_bwd(to_dev(inp.x, inp.dtype), dev["delta"], dev["A"], dev["B"], dev["C"],
                                 to_dev(dout, inp.dtype), D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"],
                                 doc_start=dev["doc_start"],
                                 initial_state=torch.from_numpy(init).cuda() if with_init else None,
                                 d_final_state=torch.from_numpy(dfin).cuda() if with_dfin else None)
    ref = oracle.selective_scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, dout, D=inp.D, z=inp.z,
                                    delta_bias=inp.delta_bias, doc_start=inp.doc_start,
                                    initial_state=init if with_init else None,
                                    d_final_state=dfin if with_dfin else None)
    compare(got, ref, inp.dtype, f"carried bwd {case} init={with_init} dfin={with_dfin}")
    if with_init:
        assert torch.count_nonzero(got["d_initial_state"][1]) == 0      # row 1 starts a document


def test_bwd_split_row_equals_whole(ssm):
    """The scan backward of a row cut in two pieces, run back to front (the second
    piece's d_initial_state is the first piece's d_final_state; its initial_state
    is the first piece's final_state from the GPU forward), gives the whole row's
    gradients; the parameter gradients are the sums of the pieces'."""
    torch = torch_mod()
    inp = make_custom(2, 900, 96, 16, dtype="f32", docs=200.0, seed=850)
    Bt, L, Dm = inp.x.shape
    dout = make_cotangent(Bt, L, Dm, dtype="f32", seed=950)
    ref = oracle.selective_scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, dout, D=inp.D, z=inp.z,
                                    delta_bias=inp.delta_bias, doc_start=inp.doc_start)
    dev = upload(inp)
    u = to_dev(inp.x, "f32")
    dy = to_dev(dout, "f32")
    cut = 389            # inside a chunk, not on a window or piece edge
    s1, s2 = slice(0, cut), slice(cut, L)
    piece = lambda sl: {k: (v[:, sl].contiguous() if k in ("delta", "B", "C", "z", "doc_start") else v)  # noqa: E731
                        for k, v in dev.items()}
    p1, p2 = piece(s1), piece(s2)
    _, h_cut = ssm.selective_scan_fwd(u[:, s1].contiguous(), p1["delta"], p1["A"], p1["B"], p1["C"], p1["D"],
                                      p1["z"], p1["delta_bias"], p1["doc_start"], final_state=True)
    g2 = ssm.selective_scan_bwd(u[:, s2].contiguous(), p2["delta"], p2["A"], p2["B"], p2["C"], dy[:, s2].contiguous(),
                                D=p2["D"], z=p2["z"], delta_bias=p2["delta_bias"], doc_start=p2["doc_start"],
                                initial_state=h_cut)
    g1 = ssm.selective_scan_bwd(u[:, s1].contiguous(), p1["delta"], p1["A"], p1["B"], p1["C"], dy[:, s1].contiguous(),
                                D=p1["D"], z=p1["z"], delta_bias=p1["delta_bias"], doc_start=p1["doc_start"],
                                d_final_state=g2["d_initial_state"])
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        assert_close(np.concatenate([to_host(g1[k]), to_host(g2[k])], axis=1), ref[k], "f32", f"split {k}")
    for k in ("dA", "dD", "ddelta_bias"):
        assert_close(to_host(g1[k]) + to_host(g2[k]), ref[k], "f32", f"split {k}")


def test_bwd_workload_carried(ssm):
    """The packed 32K workload shape with a given initial state and a gradient at
    the final state, both supported on the sampled channels' adjoints."""
    torch = torch_mod()
    inp = make_inputs("packed_32k")
    Bt, L, Dm = inp.x.shape
    N = inp.A.shape[1]
    inp.doc_start[0, 0] = 0
    ch = np.array(SAMPLES["packed_32k"])
    print(f"[bwd carried] packed_32k shape={inp.x.shape}", flush=True)
    rng = np.random.default_rng(921)
    init = rng.normal(0.0, 0.5, size=(Bt, Dm, N)).astype(np.float32)
    dfin = np.zeros((Bt, Dm, N), dtype=np.float32)
    dfin[:, ch] = rng.normal(0.0, 1.0, size=(Bt, len(ch), N))
    dout = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=922, channels=ch)
    dev = upload(inp)
    got = ssm.selective_scan_bwd(to_dev(inp.x, inp.dtype), dev["delta"], dev["A"], dev["B"], dev["C"],
                                 to_dev(dout, inp.dtype), D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"],
                                 doc_start=dev["doc_start"], initial_state=torch.from_numpy(init).cuda(),
                                 d_final_state=torch.from_numpy(dfin).cuda())
    torch.cuda.synchronize()
    idx = torch.from_numpy(ch).to(got["du"].device)
    others = torch.from_numpy(np.setdiff1d(np.arange(Dm), ch)).to(got["du"].device)
    assert torch.count_nonzero(got["d_initial_state"].index_select(1, others)) == 0
    sub = {k: to_host(got[k].index_select(2, idx)) for k in ("du", "ddelta", "dz")}
    sub.update({k: to_host(got[k].index_select(0, idx)) for k in ("dA", "dD", "ddelta_bias")})
    sub.update({k: to_host(got[k]) for k in ("dB", "dC")})
    sub["d_initial_state"] = to_host(got["d_initial_state"].index_select(1, idx))
    del dev, got
    ref = oracle.selective_scan_bwd(inp.x[:, :, ch], inp.delta[:, :, ch], inp.A[ch], inp.B, inp.C, dout[:, :, ch],
                                    D=inp.D[ch], z=inp.z[:, :, ch], delta_bias=inp.delta_bias[ch],
                                    doc_start=inp.doc_start, initial_state=init[:, ch], d_final_state=dfin[:, ch])
    for k in sorted(ref):
        assert_close(sub[k], ref[k], inp.dtype, f"carried packed_32k {k}")


CONV_HIST_CASES = [
    # (batch, seqlen, dim, dtype, docs)
    (2, 200, 64, "bf16", 20.0),       # channel pairs
    (2, 131, 37, "f32", 9.0),         # odd D: one channel a thread
    (2, 1, 24, "bf16", None),         # one token: the history gets w of taps 1..3 only
    (2, 2, 38, "f32", None),
]


@pytest.mark.parametrize("case", CONV_HIST_CASES, ids=lambda c: "x".join(map(str, c)))
def test_conv_bwd_with_history(ssm, case):
    torch = torch_mod()
    Bt, L, Dm, dt, docs = case
    inp = make_custom(Bt, L, Dm, 4, dtype=dt, docs=docs, seed=860 + L + Dm)
    inp.conv_b[:] = np.linspace(-0.3, 0.3, Dm).astype(np.float32)
    inp.doc_start[0, 0] = 0       # row 0 continues the history
    inp.doc_start[1, 0] = 1       # row 1 starts a document: zero history gradient
    if L > 2:
        inp.doc_start[0, 2] = 1   # and in row 0 a start cuts the history off token 2
    rng = np.random.default_rng(861)
    hist = rng.normal(0.0, 1.0, size=(Bt, Dm, 3)).astype(np.float32)
    if dt == "bf16":
        hist = bf16_round(hist)
    du = make_cotangent(Bt, L, Dm, dtype=dt, seed=960 + L)
    dev = upload(inp)
    got = ssm.causal_conv1d_bwd(dev["x"], dev["conv_w"], to_dev(du, dt), dev["conv_b"], dev["doc_start"],
                                conv_state=to_dev(hist, dt))
    ref = oracle.causal_conv1d_bwd(inp.x, inp.conv_w, du, inp.conv_b, inp.doc_start, conv_state=hist)
    for i, what in enumerate(("dx", "dweight", "dbias", "d_conv_state")):
        assert_close(to_host(got[i]), ref[i], dt, f"conv history {what}")
    assert torch.count_nonzero(got[3][1]) == 0


def test_conv_bwd_split_row_equals_whole(ssm):
    """Conv backward of a row cut in two: the second piece takes the first piece's
    last three inputs as history (zeroed before a document start inside them), and
    its d_conv_state adds to the first piece's dx there."""
    inp = make_custom(2, 400, 64, 4, dtype="f32", docs=30.0, seed=870)
    inp.conv_b[:] = 0.1
    cut = 150
    inp.doc_start[0, cut - 1] = 1   # row 0: a document starts inside the history window
    inp.doc_start[1, cut - 3:cut + 1] = 0
    Bt, L, Dm = inp.x.shape
    du = make_cotangent(Bt, L, Dm, dtype="f32", seed=970)
    ref = oracle.causal_conv1d_bwd(inp.x, inp.conv_w, du, inp.conv_b, inp.doc_start)
    hist = np.ascontiguousarray(inp.x[:, cut - 3:cut].transpose(0, 2, 1))
    for b in range(Bt):
        starts = np.nonzero(inp.doc_start[b, cut - 3:cut])[0]
        if starts.size:
            hist[b, :, :starts[-1]] = 0.0
    dev = upload(inp)
    s1, s2 = slice(0, cut), slice(cut, L)
    dx1, dw1, db1 = ssm.causal_conv1d_bwd(dev["x"][:, s1].contiguous(), dev["conv_w"], to_dev(du[:, s1], "f32"),
                                          dev["conv_b"], dev["doc_start"][:, s1].contiguous())
    dx2, dw2, db2, dh2 = ssm.causal_conv1d_bwd(dev["x"][:, s2].contiguous(), dev["conv_w"], to_dev(du[:, s2], "f32"),
                                               dev["conv_b"], dev["doc_start"][:, s2].contiguous(),
                                               conv_state=to_dev(hist, "f32"))
    dx = np.concatenate([to_host(dx1), to_host(dx2)], axis=1)
    dh = to_host(dh2).transpose(0, 2, 1)                         # (B, 3, D)
    for b in range(Bt):
        starts = np.nonzero(inp.doc_start[b, cut - 3:cut])[0]
        lo = starts[-1] if starts.size else 0
        dx[b, cut - 3 + lo:cut] += dh[b, lo:]
    assert_close(dx, ref[0], "f32", "split conv dx")
    assert_close(to_host(dw1) + to_host(dw2), ref[1], "f32", "split conv dweight")
    assert_close(to_host(db1) + to_host(db2), ref[2], "f32", "split conv dbias")


def test_train_step_graph_replays_match_eager(ssm):
    """The fused forward, the scan backward and the conv backward captured in one
    HIP graph (caller-owned outputs and workspaces, nothing allocated by the
    library): every replay, with eager work between replays, reproduces the
    eager results bit for bit."""
    torch = torch_mod()
    inp = make_custom(2, 1000, 128, 16, dtype="bf16", docs=150.0, seed=880)
    Bt, L, Dm = inp.x.shape
    N = inp.A.shape[1]
    dev = upload(inp)
    dout = to_dev(make_cotangent(Bt, L, Dm, dtype="bf16", seed=980), "bf16")
    ws_f = torch.empty(max(ssm.scan_workspace_bytes(Bt, L, Dm, N), 1), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(ssm.scan_bwd_workspace_bytes(Bt, L, Dm, N), dtype=torch.uint8, device="cuda")
    ws_c = torch.empty(ssm.conv_bwd_workspace_bytes(Bt, L, Dm), dtype=torch.uint8, device="cuda")
    u = torch.empty_like(dev["x"])
    out = torch.empty_like(dev["x"])
    fin = torch.empty((Bt, Dm, N), dtype=torch.float32, device="cuda")
    grads = ssm.selective_scan_bwd(u, dev["delta"], dev["A"], dev["B"], dev["C"], dout, dev["D"], dev["z"],
                                   dev["delta_bias"], dev["doc_start"], workspace=ws_b)
    dx = torch.empty_like(dev["x"])
    dw = torch.empty((Dm, 4), dtype=torch.float32, device="cuda")
    db = torch.empty((Dm,), dtype=torch.float32, device="cuda")

    def step():
        ssm.conv_scan_fwd(dev["x"], dev["conv_w"], dev["conv_b"], dev["delta"], dev["A"], dev["B"], dev["C"],
                          dev["D"], dev["z"], dev["delta_bias"], dev["doc_start"], u=u, out=out, final_state=fin,
                          workspace=ws_f)
        ssm.selective_scan_bwd(u, dev["delta"], dev["A"], dev["B"], dev["C"], dout, dev["D"], dev["z"],
                               dev["delta_bias"], dev["doc_start"], workspace=ws_b, grads=grads)
        ssm.causal_conv1d_bwd(dev["x"], dev["conv_w"], grads["du"], dev["conv_b"], dev["doc_start"],
                              workspace=ws_c, dx=dx, dweight=dw, dbias=db)

    results = lambda: [t.clone() for t in (u, out, fin, dx, dw, db)] + [grads[k].clone() for k in sorted(grads)]  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref = results()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (u, out, fin, dx, dw, db, *grads.values()):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert torch.equal(a, b), f"replay {rep}: result {i}"
        _ = (out.float() * 2).sum().item()      # eager work between replays


@pytest.mark.parametrize("case", ["A_zero", "step_to_zero", "large_step"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_degenerate_parameters(ssm, case, dtype):
    """The method's degenerate cases, backward: A = 0 (the state is a running
    sum), a vanishing step (delta_bias = -60: softplus ~ 1e-26, only the skip
    and gate terms carry gradient) and a large step (delta_bias = +5: decays
    down to e^-5 and below, each token nearly forgets the last)."""
    inp = make_custom(2, 700, 96, 16, dtype=dtype, docs=150.0, seed=890)
    if case == "A_zero":
        inp.A[:] = 0.0
    elif case == "step_to_zero":
        inp.delta_bias[:] = -60.0
    else:
        inp.delta_bias[:] = 5.0
    bwd_case(ssm, inp, seed=990)
