"""GPU test of mamba_selective_scan_fwd_noalloc: the allocation-free scan gives
the results of mamba_selective_scan_fwd (with its caller-provided workspace) on
two calls in a row, the second on a smaller input, for per-channel A and both
scalar-A-heads forms.  With fp32 I/O the two entry points run the same
arithmetic and must agree bit for bit; with bf16 I/O the workspace entry point
rounds its handed-over step sizes to bf16, so the two agree to the bf16
tolerance of the path."""

import numpy as np
import pytest

from gpu_helpers import TOL, assert_close, to_host, upload
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _run_pair(ssm, torch, inp, dev, with_init):
    t = upload(inp, dev)
    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    u = ssm.causal_conv1d_fwd(t["x"], t["conv_w"], t["conv_b"], t["doc_start"])
    init = None
    if with_init:
        g = torch.Generator(device="cpu").manual_seed(L)
        init = torch.randn((B, D, N), generator=g, dtype=torch.float32).to(dev)
    ref_out, ref_fin = ssm.selective_scan_fwd(u, t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                              t["delta_bias"], t["doc_start"], initial_state=init)
    out = torch.full_like(u, float("nan"))
    fin = torch.full((B, D, N), float("nan"), dtype=torch.float32, device=dev)
    ssm.selective_scan_fwd_noalloc(u, t["delta"], t["A"], t["B"], t["C"], out, t["D"], t["z"], t["delta_bias"],
                                   t["doc_start"], final_state=fin, initial_state=init)
    torch.cuda.synchronize()
    return to_host(out), to_host(fin), to_host(ref_out), to_host(ref_fin)


@pytest.mark.parametrize("kind", ["channels_bf16", "channels_f32", "heads_bf16", "heads_f32"])
def test_noalloc_matches_workspace_entry(kind):
    torch = pytest.importorskip("torch")
    import selective_state_space_23_amd as ssm
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    dev = torch.device("cuda:0")
    dtype = "f32" if kind.endswith("f32") else "bf16"
    if kind.startswith("channels"):
        shapes = [dict(batch=2, seqlen=9000, dim=448, dstate=16), dict(batch=1, seqlen=1300, dim=200, dstate=8)]
    else:
        shapes = [dict(batch=2, seqlen=3000, dim=256, dstate=64, nheads=4),
                  dict(batch=1, seqlen=700, dim=128, dstate=32, nheads=2)]
    # two calls in a row, the second with a smaller input: the array keeps the
    # first call's carries, which the second must not read
    for i, shp in enumerate(shapes):
        inp = make_custom(dtype=dtype, docs=800.0, seed=100 + i, **shp)
        print(f"noalloc {kind} call {i}: {shp}", flush=True)
        got, gfin, ref, rfin = _run_pair(ssm, torch, inp, dev, with_init=(i == 1))
        if dtype == "f32":
            assert np.array_equal(got, ref), f"{kind} call {i}: out differs from the workspace entry point"
            assert np.array_equal(gfin, rfin), f"{kind} call {i}: final_state differs"
        else:
            assert_close(got, ref, "bf16", f"{kind} call {i} out")
            assert_close(gfin, rfin, "bf16", f"{kind} call {i} final_state")
    assert TOL["bf16"] == (2e-2, 2e-2)
