"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element; they span several 64-token scan
chunks, ragged channel counts (not a multiple of 64 or of the conv vector
width), ragged token tails and the method's degenerate cases.  The five named
workloads run at full size in the same launch configuration as the benchmark;
there the oracle recomputes sampled channels over the whole sequence (chains are
independent per channel, so a sampled channel is exact, not approximate)."""

import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_custom, make_inputs

from gpu_helpers import (assert_close, oracle_pipeline, oracle_scan, to_dev, to_host, torch_mod,
                         upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (they fail instead of skipping)")
    import selective_state_space_23_amd as mod
    mod._lib.load()
    return mod


def run_conv(ssm, dev, inp, apply_silu=True, use_bias=True, use_docs=True):
    return ssm.causal_conv1d_fwd(dev["x"], dev["conv_w"], dev["conv_b"] if use_bias else None,
                                 dev["doc_start"] if use_docs else None, apply_silu=apply_silu)


def run_scan(ssm, dev, u, use_z=True, use_D=True, use_bias=True, softplus=True, final_state=True,
             initial_state=None):
    return ssm.selective_scan_fwd(u, dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"] if use_D else None,
                                  dev["z"] if use_z else None, dev["delta_bias"] if use_bias else None,
                                  dev["doc_start"], delta_softplus=softplus, final_state=final_state,
                                  initial_state=initial_state)


# ----------------------------------------------------------------------------
# causal conv1d
# ----------------------------------------------------------------------------
CONV_CASES = [
    # (batch, seqlen, dim, dtype, docs)
    (1, 64, 16, "f32", None),
    (2, 200, 64, "bf16", 20.0),      # vectorised bf16 path, several 48-token tiles
    (2, 131, 37, "bf16", 9.0),       # ragged D -> per-channel path
    (1, 100, 36, "f32", 7.0),        # ragged D for f32 vectors
    (3, 1, 24, "bf16", None),        # one token
    (2, 3, 24, "bf16", 2.0),         # fewer tokens than the conv width
    (1, 1000, 1536, "bf16", 64.0),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("silu,bias", [(True, True), (False, False)])
def test_conv_parity_small(ssm, case, silu, bias):
    Bt, L, Dm, dt, docs = case
    inp = make_custom(Bt, L, Dm, 4, dtype=dt, docs=docs, seed=100 + L + Dm)
    inp.conv_b[:] = np.linspace(-0.3, 0.3, Dm).astype(np.float32)
    dev = upload(inp)
    got = to_host(run_conv(ssm, dev, inp, apply_silu=silu, use_bias=bias))
    ref = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b if bias else None, inp.doc_start, apply_silu=silu)
    assert_close(got, ref, dt, f"conv {case}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_document_edges(ssm, dtype):
    """Starts on every token, and just before/at/after the 48-token tile edges."""
    inp = make_custom(3, 150, 64, 4, dtype=dtype, docs=None, seed=7)
    inp.doc_start[0, :] = 1
    for t in (44, 45, 46, 47, 48, 49, 50, 51, 95, 96, 97, 144):
        inp.doc_start[1, t] = 1
    inp.doc_start[2, 1] = 1
    inp.doc_start[2, 2] = 1
    dev = upload(inp)
    got = to_host(run_conv(ssm, dev, inp))
    ref = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    assert_close(got, ref, dtype, "conv doc edges")
    no_docs = to_host(run_conv(ssm, dev, inp, use_docs=False))
    assert_close(no_docs, oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, None), dtype, "conv no docs")


# ----------------------------------------------------------------------------
# selective scan on small shapes
# ----------------------------------------------------------------------------
def scan_case(ssm, inp, **flags):
    """GPU scan on u = bf16(oracle conv(x)) vs the oracle scan on the same u."""
    u = oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start)
    u32 = bf16_round(u.astype(np.float32)) if inp.dtype == "bf16" else u.astype(np.float32)
    dev = upload(inp)
    gflags = dict(flags)
    if flags.get("initial_state") is not None:
        gflags["initial_state"] = torch_mod().from_numpy(flags["initial_state"].astype(np.float32)).cuda()
    out, fin = run_scan(ssm, dev, to_dev(u32, inp.dtype), **gflags)
    ch = np.arange(inp.x.shape[2])
    kw = {k: v for k, v in flags.items() if k != "final_state"}
    ref_out, ref_fin = oracle_scan(inp, u32.astype(np.float64), ch, **kw)
    assert_close(to_host(out), ref_out, inp.dtype, "scan out")
    if fin is not None:
        assert_close(to_host(fin), ref_fin, inp.dtype, "scan final_state")
    return out, fin


SCAN_CASES = [
    # (batch, seqlen, dim, dstate, nheads, dtype, docs)
    (1, 64, 16, 4, 0, "f32", None),
    (2, 1000, 100, 16, 0, "bf16", 150.0),    # 7 chunks of 128 with a 104-token tail, ragged D
    (2, 777, 64, 8, 0, "bf16", 90.0),
    (1, 500, 70, 4, 0, "f32", 60.0),
    (3, 257, 130, 16, 0, "f32", 40.0),
    (1, 300, 128, 16, 2, "bf16", 70.0),      # heads, headdim 64
    (1, 300, 128, 32, 4, "bf16", 70.0),      # heads, headdim 32: one wave spans two heads
    (2, 200, 128, 64, 2, "f32", 50.0),
    (1, 260, 192, 128, 3, "bf16", 80.0),
    (1, 333, 64, 8, 2, "bf16", 40.0),        # heads: headdim 32, 8 states (padded to 32 in the products)
    (2, 450, 128, 24, 2, "bf16", 60.0),      # heads: 24 states
    (1, 200, 64, 128, 2, "bf16", 30.0),      # heads: headdim 32, 128 states
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_scan_parity_small(ssm, case):
    Bt, L, Dm, N, H, dt, docs = case
    inp = make_custom(Bt, L, Dm, N, nheads=H, dtype=dt, docs=docs, seed=200 + L)
    scan_case(ssm, inp)


@pytest.mark.parametrize("flags", [
    dict(use_z=False), dict(use_D=False), dict(use_bias=False), dict(softplus=False, use_bias=False),
    dict(final_state=False), dict(use_z=False, use_D=False, use_bias=False)], ids=str)
def test_scan_optional_arguments(ssm, flags):
    inp = make_custom(2, 333, 96, 16, dtype="bf16", docs=100.0, seed=301)
    if flags.get("softplus") is False:
        inp.delta[:] = bf16_round(np.abs(inp.delta) * 0.5 + 0.01)     # positive raw steps
    scan_case(ssm, inp, **flags)


def test_scan_single_token_and_every_token_a_document(ssm):
    inp = make_custom(2, 1, 64, 16, dtype="f32", docs=None, seed=302)
    scan_case(ssm, inp)
    inp = make_custom(1, 190, 64, 16, dtype="f32", docs=None, seed=303)
    inp.doc_start[:] = 1
    scan_case(ssm, inp)


def test_scan_documents_at_chunk_edges(ssm):
    inp = make_custom(2, 400, 64, 16, dtype="f32", docs=None, seed=304)
    for t in (63, 64, 65, 127, 128, 192, 256, 320, 399):
        inp.doc_start[0, t] = 1
    inp.doc_start[1, 64::64] = 1
    scan_case(ssm, inp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_heads_documents_at_chunk_edges(ssm, dtype):
    """Scalar-A heads: starts on either side of the 64-token chunk edges, a row with
    a start on every token, and a row with none."""
    inp = make_custom(3, 400, 128, 32, nheads=2, dtype=dtype, docs=None, seed=310)
    for t in (1, 62, 63, 64, 65, 127, 128, 129, 255, 256, 320, 399):
        inp.doc_start[0, t] = 1
    inp.doc_start[1, :] = 1
    scan_case(ssm, inp)


def test_heads_f32_n128_window_edges(ssm):
    """fp32 scalar-A heads at N = 128 stage B and C 32 tokens at a time in the
    output pass: document starts on either side of those window edges and of the
    chunk edges, a carried state, a row length that ends mid-window."""
    inp = make_custom(2, 1331, 128, 128, nheads=2, dtype="f32", docs=None, seed=315)
    inp.doc_start[:] = 0
    for t in (31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 500, 1023, 1024, 1025, 1300):
        inp.doc_start[0, t] = 1
    inp.doc_start[1, 7::37] = 1
    init = (0.5 * np.random.default_rng(316).standard_normal((2, 128, 128))).astype(np.float32)
    scan_case(ssm, inp, initial_state=init, final_state=True)


INIT_CASES = [
    # (dim, dstate, nheads, dtype): both A layouts, both dtypes, and the matrix-core form
    (96, 16, 0, "bf16"), (64, 8, 0, "f32"), (128, 32, 2, "bf16"), (128, 16, 2, "f32"), (128, 128, 2, "bf16"),
]


@pytest.mark.parametrize("case", INIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_scan_initial_state(ssm, case):
    """A given state before token 0: row 0 continues it, row 1 starts a document at
    token 0 (and so ignores it); lengths span one chunk and several."""
    Dm, N, H, dt = case
    for L in (50, 700):
        inp = make_custom(2, L, Dm, N, nheads=H, dtype=dt, docs=120.0, seed=400 + L + N)
        inp.doc_start[0, 0] = 0
        inp.doc_start[1, 0] = 1
        init = np.random.default_rng(401).normal(0.0, 0.5, size=(2, Dm, N))
        scan_case(ssm, inp, initial_state=init)


def test_scan_split_equals_whole(ssm):
    """Scanning [0, L1) and then [L1, L) from the first part's final state gives the
    whole scan's outputs and final state (the carry a sequence-parallel split uses)."""
    torch = torch_mod()
    for H, N in ((0, 16), (2, 64)):
        inp = make_custom(2, 900, 128, N, nheads=H, dtype="bf16", docs=200.0, seed=402 + N)
        u = bf16_round(oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start).astype(np.float32))
        ch = np.arange(128)
        ref_out, ref_fin = oracle_scan(inp, u.astype(np.float64), ch)
        dev = upload(inp)
        ud = to_dev(u, "bf16")
        L1 = 333
        parts = []
        fin = None
        for sl in (slice(0, L1), slice(L1, 900)):
            sub = {k: (v[:, sl].contiguous() if k in ("delta", "B", "C", "z", "doc_start") else v) for k, v in dev.items()}
            o, fin = run_scan(ssm, sub, ud[:, sl].contiguous(), initial_state=fin)
            parts.append(to_host(o))
        assert_close(np.concatenate(parts, axis=1), ref_out, "bf16", f"split out H={H}")
        assert_close(to_host(fin), ref_fin, "bf16", f"split final_state H={H}")


def test_scan_A_zero_and_vanishing_step(ssm):
    inp = make_custom(1, 300, 64, 16, dtype="f32", docs=50.0, seed=305)
    inp.A[:] = 0.0
    scan_case(ssm, inp)
    inp = make_custom(1, 300, 64, 16, dtype="f32", docs=50.0, seed=306)
    inp.delta_bias[:] = -60.0
    out, fin = scan_case(ssm, inp)
    assert float(np.abs(to_host(fin)).max()) < 1e-20


def test_scan_large_step_forgets(ssm):
    """Large dt drives exp(dt A) to 0: the state is the last input only."""
    inp = make_custom(1, 200, 64, 16, dtype="f32", docs=None, seed=307)
    inp.delta_bias[:] = 30.0
    scan_case(ssm, inp)


def test_scan_is_deterministic(ssm):
    inp = make_custom(2, 3000, 192, 16, dtype="bf16", docs=300.0, seed=308)
    u = bf16_round(oracle.causal_conv1d(inp.x, inp.conv_w, inp.conv_b, inp.doc_start).astype(np.float32))
    dev = upload(inp)
    ud = to_dev(u, "bf16")
    o1, f1 = run_scan(ssm, dev, ud)
    o2, f2 = run_scan(ssm, dev, ud)
    torch = torch_mod()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


# ----------------------------------------------------------------------------
# Full-size workloads, sampled channels
# ----------------------------------------------------------------------------
SAMPLES = {
    "tiny_f32": None,                                   # all channels
    "m130_2k": [0, 1, 63, 64, 511, 1000, 1535],
    "packed_32k": [0, 5, 63, 64, 700, 1471, 1535],
    "wide_64k": [0, 63, 64, 2047, 4000, 5119],
    "heads_32k": [0, 63, 64, 700, 1535],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_workload_parity(ssm, name):
    inp = make_inputs(name)
    Dm = inp.x.shape[2]
    ch = np.arange(Dm) if SAMPLES[name] is None else np.array(SAMPLES[name])
    print(f"[parity] {name} shape={inp.shape} channels={ch.tolist()[:8]}", flush=True)
    dev = upload(inp)
    u_dev = run_conv(ssm, dev, inp)
    out, fin = run_scan(ssm, dev, u_dev)
    torch = torch_mod()
    torch.cuda.synchronize()
    idx = torch.from_numpy(ch).to(u_dev.device)
    u_g = to_host(u_dev.index_select(2, idx))
    out_g = to_host(out.index_select(2, idx))
    fin_g = to_host(fin.index_select(1, idx))
    del dev, u_dev, out, fin
    u_ref, out_ref, fin_ref = oracle_pipeline(inp, ch)
    u_exact = oracle.causal_conv1d(inp.x[:, :, ch], inp.conv_w[ch], inp.conv_b[ch], inp.doc_start)
    assert_close(u_g, u_exact, inp.dtype, f"{name} conv")
    assert_close(out_g, out_ref, inp.dtype, f"{name} out")
    assert_close(fin_g, fin_ref, inp.dtype, f"{name} final_state")
