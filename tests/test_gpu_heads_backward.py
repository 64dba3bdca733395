"""GPU parity of the scalar-A heads backward (Mamba-2 shape: A (H,), delta
(B, L, H), delta_bias (H,)) against the oracle's gradients, which sum the
per-channel adjoint over the channels of each head (tied parameters; pinned by
central finite differences in test_oracle_pins.py)."""

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


def run(ssm, inp, dout, init=None, dfin=None, channels=None):
    torch = torch_mod()
    dev = upload(inp)
    return ssm.selective_scan_bwd(to_dev(inp.x, inp.dtype), dev["delta"], dev["A"], dev["B"], dev["C"],
                                  to_dev(dout, inp.dtype), D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"],
                                  doc_start=dev["doc_start"],
                                  initial_state=None if init is None else torch.from_numpy(init).cuda(),
                                  d_final_state=None if dfin is None else torch.from_numpy(dfin).cuda())


def reference(inp, dout, init=None, dfin=None):
    return oracle.selective_scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, dout, D=inp.D, z=inp.z,
                                     delta_bias=inp.delta_bias, doc_start=inp.doc_start, initial_state=init,
                                     d_final_state=dfin)


def compare(got, ref, dtype, what):
    assert set(got) == set(ref), (what, sorted(got), sorted(ref))
    for k in sorted(ref):
        assert_close(to_host(got[k]), ref[k], dtype, f"{what} {k}")


CASES = [
    # (batch, seqlen, dim, nheads, dstate, dtype, docs)
    (2, 300, 128, 2, 64, "bf16", 70.0),      # one-chunk segments: every chunk joined by the carries
    (1, 500, 64, 2, 16, "f32", 100.0),       # head size 32
    (2, 333, 128, 2, 128, "f32", 90.0),      # N = 128, a ragged last chunk
    (4, 1000, 768, 12, 32, "bf16", 150.0),   # segments of several chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_heads_bwd_parity(ssm, case):
    Bt, L, Dm, H, N, dt, docs = case
    inp = make_custom(Bt, L, Dm, N, nheads=H, dtype=dt, docs=docs, seed=1600 + L + N)
    dout = make_cotangent(Bt, L, Dm, dtype=dt, seed=1700 + L)
    print(f"[heads bwd] {case}", flush=True)
    compare(run(ssm, inp, dout), reference(inp, dout), dt, f"heads bwd {case}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_heads_bwd_carried_state(ssm, dt):
    """initial_state and d_final_state: row 0 continues the carried state, row 1
    starts a document at token 0 (its d_initial_state is zero)."""
    torch = torch_mod()
    inp = make_custom(2, 400, 128, 32, nheads=2, dtype=dt, docs=120.0, seed=1800)
    inp.doc_start[:, 0] = 0
    inp.doc_start[1, 0] = 1
    rng = np.random.default_rng(1801)
    init = (0.3 * rng.standard_normal((2, 128, 32))).astype(np.float32)
    dfin = (0.3 * rng.standard_normal((2, 128, 32))).astype(np.float32)
    dout = make_cotangent(2, 400, 128, dtype=dt, seed=1802)
    got = run(ssm, inp, dout, init, dfin)
    compare(got, reference(inp, dout, init, dfin), dt, "heads bwd carried")
    assert torch.count_nonzero(got["d_initial_state"][1]) == 0


@pytest.mark.parametrize("N", [20, 100])
def test_heads_bwd_padded_states(ssm, N):
    """N not a multiple of 16: the kernels run on zero-padded copies."""
    inp = make_custom(2, 260, 128, N, nheads=2, dtype="bf16", docs=80.0, seed=1900 + N)
    dout = make_cotangent(2, 260, 128, dtype="bf16", seed=1901 + N)
    compare(run(ssm, inp, dout), reference(inp, dout), "bf16", f"heads bwd N={N}")


def test_heads_bwd_is_deterministic(ssm):
    torch = torch_mod()
    inp = make_custom(2, 700, 256, 64, nheads=4, dtype="bf16", docs=200.0, seed=2000)
    dout = make_cotangent(2, 700, 256, dtype="bf16", seed=2001)
    g1 = run(ssm, inp, dout)
    g2 = run(ssm, inp, dout)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_heads_bwd_workload(ssm):
    """The 32K heads shape (2 x 32768 tokens, 24 heads of 64 channels, N = 128) at
    full size, with the cotangent on head 5 only: every gradient of head 5 and dB,
    dC (which then come from head 5 alone) against the oracle on that head's
    channels; the other heads' du and ddelta must be zero."""
    torch = torch_mod()
    inp = make_inputs("heads_32k")
    Bt, L, Dm = inp.x.shape
    H, P, hsel = inp.nheads, Dm // inp.nheads, 5
    ch = np.arange(hsel * P, (hsel + 1) * P)
    dout = make_cotangent(Bt, L, Dm, dtype=inp.dtype, seed=2100, channels=ch)
    print("[heads bwd] heads_32k full size", flush=True)
    got = run(ssm, inp, dout)
    torch.cuda.synchronize()
    sub = make_custom(1, 1, P, inp.B.shape[-1], nheads=1, dtype=inp.dtype, seed=0)
    sub.x, sub.z, sub.D = inp.x[:, :, ch], inp.z[:, :, ch], inp.D[ch]
    sub.delta, sub.delta_bias, sub.A = inp.delta[:, :, hsel:hsel + 1], inp.delta_bias[hsel:hsel + 1], inp.A[hsel:hsel + 1]
    sub.B, sub.C, sub.doc_start = inp.B, inp.C, inp.doc_start
    ref = reference(sub, dout[:, :, ch])
    assert_close(to_host(got["du"][:, :, ch]), ref["du"], "bf16", "heads_32k du")
    assert_close(to_host(got["dz"][:, :, ch]), ref["dz"], "bf16", "heads_32k dz")
    assert_close(to_host(got["dD"][ch]), ref["dD"], "bf16", "heads_32k dD")
    assert_close(to_host(got["ddelta"][:, :, hsel:hsel + 1]), ref["ddelta"], "bf16", "heads_32k ddelta")
    assert_close(to_host(got["dA"][hsel:hsel + 1]), ref["dA"], "bf16", "heads_32k dA")
    assert_close(to_host(got["ddelta_bias"][hsel:hsel + 1]), ref["ddelta_bias"], "bf16", "heads_32k ddelta_bias")
    assert_close(to_host(got["dB"]), ref["dB"], "bf16", "heads_32k dB")
    assert_close(to_host(got["dC"]), ref["dC"], "bf16", "heads_32k dC")
    others = np.setdiff1d(np.arange(Dm), ch)
    assert float(got["du"][:, :, torch.from_numpy(others).cuda()].abs().max()) == 0.0
    assert float(got["ddelta"][:, :, [h for h in range(H) if h != hsel]].abs().max()) == 0.0


@pytest.mark.parametrize("flags", [
    dict(use_z=False), dict(use_D=False), dict(use_bias=False), dict(softplus=False, use_bias=False),
    dict(use_docs=False), dict(use_z=False, use_D=False, use_bias=False),
], ids=lambda f: ",".join(f"{k}={v}" for k, v in f.items()))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_heads_bwd_optional_inputs(ssm, flags, dt):
    """z, D, delta_bias, the softplus and doc_start each absent: the gradients the
    absent inputs would have are not returned, the others match the oracle."""
    torch = torch_mod()
    use_z, use_D = flags.get("use_z", True), flags.get("use_D", True)
    use_bias, softplus = flags.get("use_bias", True), flags.get("softplus", True)
    use_docs = flags.get("use_docs", True)
    inp = make_custom(2, 450, 128, 32, nheads=2, dtype=dt, docs=110.0, seed=1950)
    if not softplus:
        # delta is the step size itself: positive ones (negative steps make the
        # decays exceed 1 and the gradient sums ill-conditioned)
        pos = np.abs(inp.delta) * np.float32(0.5) + np.float32(0.001)
        inp.delta[:] = bf16_round(pos) if dt == "bf16" else pos
    dout = make_cotangent(2, 450, 128, dtype=dt, seed=1951)
    print(f"[heads bwd] optional {flags} {dt}", flush=True)
    dev = upload(inp)
    got = ssm.selective_scan_bwd(to_dev(inp.x, dt), dev["delta"], dev["A"], dev["B"], dev["C"], to_dev(dout, dt),
                                 D=dev["D"] if use_D else None, z=dev["z"] if use_z else None,
                                 delta_bias=dev["delta_bias"] if use_bias else None,
                                 doc_start=dev["doc_start"] if use_docs else None, delta_softplus=softplus)
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(inp.x, inp.delta, inp.A, inp.B, inp.C, dout, D=inp.D if use_D else None,
                                    z=inp.z if use_z else None, delta_bias=inp.delta_bias if use_bias else None,
                                    delta_softplus=softplus, doc_start=inp.doc_start if use_docs else None)
    compare(got, ref, dt, f"heads bwd {flags}")


def test_heads_bwd_documents_at_chunk_edges(ssm):
    """Documents starting on 16-token chunk boundaries, one token before and after
    them, on segment boundaries, and one-token documents."""
    inp = make_custom(2, 1100, 128, 64, nheads=2, dtype="f32", docs=None, seed=1960)
    inp.doc_start[:] = 0
    inp.doc_start[:, 0] = 1
    for t in (15, 16, 17, 31, 32, 33, 47, 48, 256, 257, 511, 512, 513, 514, 1024, 1099):
        inp.doc_start[0, t] = 1
    for t in range(40, 1100, 53):
        inp.doc_start[1, t] = 1
    dout = make_cotangent(2, 1100, 128, dtype="f32", seed=1961)
    print("[heads bwd] documents at chunk edges", flush=True)
    compare(run(ssm, inp, dout), reference(inp, dout), "f32", "heads bwd doc edges")
