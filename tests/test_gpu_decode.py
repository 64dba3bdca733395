"""GPU parity of the one-token decode steps (conv window update + recurrence step)
against the fp64 oracle run over the whole sequence at once: generating token by
token must give the same outputs and final state as scanning the sequence."""

import numpy as np
import pytest

from workloads import make_custom

from gpu_helpers import assert_close, oracle_pipeline, to_dev, to_host, torch_mod, upload

pytestmark = pytest.mark.gpu

CASES = [
    # (dim, dstate, nheads, dtype)
    (96, 16, 0, "bf16"), (40, 4, 0, "f32"), (128, 128, 2, "bf16"), (128, 64, 4, "f32"), (64, 8, 0, "bf16"),
]


@pytest.fixture(scope="module")
def ssm():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (they fail instead of skipping)")
    import selective_state_space_23_amd as mod
    mod._lib.load()
    return mod


def conv_window(x, doc_start, t):
    """Conv history entering token t: x[t-3 .. t-1], zero before the latest document
    start at or before t-1 (and before token 0)."""
    Bt, _, Dm = x.shape
    w = np.zeros((Bt, Dm, 3), dtype=np.float32)
    for b in range(Bt):
        first = 0
        for s in range(max(t - 3, 0), t):
            if doc_start[b, s]:
                first = s
        for k, s in enumerate(range(t - 3, t)):
            if s >= max(first, 0) and s >= 0:
                w[b, :, k] = x[b, s]
    return w


def step_all(ssm, inp, dev, t_from, t_to, conv_state, state):
    """Run decode steps for tokens t_from .. t_to-1; returns outputs (B, steps, D)."""
    torch = torch_mod()
    outs = []
    for t in range(t_from, t_to):
        reset = dev["doc_start"][:, t].contiguous()
        if t == 0:
            reset = torch.ones_like(reset)
        u_t = ssm.causal_conv1d_update(dev["x"][:, t].contiguous(), conv_state, dev["conv_w"], dev["conv_b"],
                                       reset=reset)
        o = ssm.selective_state_update(state, u_t, dev["delta"][:, t].contiguous(), dev["A"],
                                       dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous(), dev["D"],
                                       dev["z"][:, t].contiguous(), dev["delta_bias"], reset=reset)
        outs.append(to_host(o))
    return np.stack(outs, axis=1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_from_scratch(ssm, case):
    torch = torch_mod()
    Dm, N, H, dt = case
    inp = make_custom(2, 40, Dm, N, nheads=H, dtype=dt, docs=9.0, seed=500 + Dm + N)
    inp.conv_b[:] = np.linspace(-0.2, 0.2, Dm).astype(np.float32)
    dev = upload(inp)
    conv_state = torch.zeros((2, Dm, 3), dtype=dev["x"].dtype, device="cuda")
    state = torch.zeros((2, Dm, N), dtype=torch.float32, device="cuda")
    got = step_all(ssm, inp, dev, 0, 40, conv_state, state)
    _, ref_out, ref_fin = oracle_pipeline(inp, np.arange(Dm))
    assert_close(got, ref_out, dt, f"decode out {case}")
    assert_close(to_host(state), ref_fin, dt, f"decode state {case}")


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "x".join(map(str, c)))
def test_prefill_then_decode(ssm, case):
    """Prefill 150 tokens with the chunked kernels, then decode 20 more."""
    torch = torch_mod()
    Dm, N, H, dt = case
    T, L0 = 170, 150
    inp = make_custom(2, T, Dm, N, nheads=H, dtype=dt, docs=30.0, seed=600 + Dm + N)
    inp.doc_start[0, L0 - 2] = 1          # a document starts inside the handed-over conv window
    dev = upload(inp)
    pre = {k: (v[:, :L0].contiguous() if k in ("x", "z", "delta", "B", "C", "doc_start") else v)
           for k, v in dev.items()}
    u = ssm.causal_conv1d_fwd(pre["x"], pre["conv_w"], pre["conv_b"], pre["doc_start"])
    out_pre, state = ssm.selective_scan_fwd(u, pre["delta"], pre["A"], pre["B"], pre["C"], pre["D"], pre["z"],
                                            pre["delta_bias"], pre["doc_start"])
    conv_state = to_dev(conv_window(inp.x, inp.doc_start, L0), dt)
    got = step_all(ssm, inp, dev, L0, T, conv_state, state)
    _, ref_out, ref_fin = oracle_pipeline(inp, np.arange(Dm))
    assert_close(to_host(out_pre), ref_out[:, :L0], dt, f"prefill out {case}")
    assert_close(got, ref_out[:, L0:], dt, f"decode out {case}")
    assert_close(to_host(state), ref_fin, dt, f"decode state {case}")


def test_decode_graph_replays_match_eager(ssm):
    """Decode steps captured in a HIP graph (as bench.py --path decode replays
    them): every replay, with eager work and synchronisations between replays,
    gives the eager outputs and states bit for bit."""
    torch = torch_mod()
    inp = make_custom(2, 40, 96, 16, dtype="bf16", docs=9.0, seed=321)
    dev = upload(inp)
    T = 12
    xs = dev["x"][:, :T].transpose(0, 1).contiguous()
    zs = dev["z"][:, :T].transpose(0, 1).contiguous()
    dls = dev["delta"][:, :T].transpose(0, 1).contiguous()
    Bs = dev["B"][:, :T].transpose(0, 1).contiguous()
    Cs = dev["C"][:, :T].transpose(0, 1).contiguous()
    rs = dev["doc_start"][:, :T].transpose(0, 1).contiguous()
    rs[0].fill_(1)
    state = torch.zeros((2, 96, 16), dtype=torch.float32, device="cuda")
    cstate = torch.zeros((2, 96, 3), dtype=torch.bfloat16, device="cuda")
    us = torch.empty((T, 2, 96), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty_like(us)

    def steps():
        for k in range(T):
            ssm.causal_conv1d_update(xs[k], cstate, dev["conv_w"], dev["conv_b"], reset=rs[k], out=us[k])
            ssm.selective_state_update(state, us[k], dls[k], dev["A"], Bs[k], Cs[k], dev["D"], zs[k],
                                       dev["delta_bias"], reset=rs[k], out=outs[k])

    # eager reference from a fixed starting state
    start_state = torch.randn((2, 96, 16), dtype=torch.float32, device="cuda") * 0.1
    start_conv = (torch.randn((2, 96, 3), device="cuda") * 0.5).to(torch.bfloat16)
    state.copy_(start_state)
    cstate.copy_(start_conv)
    steps()
    ref_out, ref_state, ref_conv = outs.clone(), state.clone(), cstate.clone()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        steps()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            steps()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(start_state)
        cstate.copy_(start_conv)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_out), f"replay {rep}: outputs"
        assert torch.equal(state, ref_state), f"replay {rep}: state"
        assert torch.equal(cstate, ref_conv), f"replay {rep}: conv window"
        _ = (outs.float() * 2).sum().item()      # eager work between replays


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_fused_decode_step_matches_two_steps(ssm, case):
    """mamba_conv_state_update (one launch) gives, bit for bit, the outputs, u,
    states and conv windows of mamba_causal_conv1d_update followed by
    mamba_selective_state_update, over steps with document starts."""
    torch = torch_mod()
    Dm, N, H, dt = case
    inp = make_custom(2, 30, Dm, N, nheads=H, dtype=dt, docs=7.0, seed=400 + Dm + N)
    dev = upload(inp)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    st1 = torch.randn((2, Dm, N), dtype=torch.float32, device="cuda") * 0.1
    cs1 = (torch.randn((2, Dm, 3), device="cuda") * 0.5).to(tdt)
    st2, cs2 = st1.clone(), cs1.clone()
    for t in range(30):
        reset = dev["doc_start"][:, t].contiguous()
        args = (dev["delta"][:, t].contiguous(), dev["A"], dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous(),
                dev["D"], dev["z"][:, t].contiguous(), dev["delta_bias"])
        x_t = dev["x"][:, t].contiguous()
        u1 = ssm.causal_conv1d_update(x_t, cs1, dev["conv_w"], dev["conv_b"], reset=reset)
        o1 = ssm.selective_state_update(st1, u1, *args, reset=reset)
        u2 = torch.empty_like(u1)
        o2 = ssm.conv_state_update(x_t, cs2, dev["conv_w"], dev["conv_b"], st2, *args, reset=reset, u_out=u2)
        torch.cuda.synchronize()
        assert torch.equal(u1, u2), f"u at token {t}"
        assert torch.equal(o1, o2), f"out at token {t}"
        assert torch.equal(st1, st2), f"state at token {t}"
        assert torch.equal(cs1, cs2), f"conv window at token {t}"


@pytest.mark.parametrize("Dm", [1536, 5120])
def test_decode_model_widths(ssm, Dm):
    """The fused one-token step at the model widths of the workloads (mamba-130m's
    1536 channels, mamba-2.8b's 5120), N = 16, from a zero state over 24 tokens
    with document starts, against the oracle on every channel."""
    torch = torch_mod()
    inp = make_custom(2, 24, Dm, 16, dtype="bf16", docs=8.0, seed=450 + Dm)
    dev = upload(inp)
    conv_state = torch.zeros((2, Dm, 3), dtype=dev["x"].dtype, device="cuda")
    state = torch.zeros((2, Dm, 16), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(24):
        reset = dev["doc_start"][:, t].contiguous()
        if t == 0:
            reset = torch.ones_like(reset)
        o = ssm.conv_state_update(dev["x"][:, t].contiguous(), conv_state, dev["conv_w"], dev["conv_b"], state,
                                  dev["delta"][:, t].contiguous(), dev["A"], dev["B"][:, t].contiguous(),
                                  dev["C"][:, t].contiguous(), dev["D"], dev["z"][:, t].contiguous(),
                                  dev["delta_bias"], reset=reset)
        outs.append(to_host(o))
    _, ref_out, ref_fin = oracle_pipeline(inp, np.arange(Dm))
    assert_close(np.stack(outs, axis=1), ref_out, "bf16", f"decode out D={Dm}")
    assert_close(to_host(state), ref_fin, "bf16", f"decode state D={Dm}")
