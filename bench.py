#!/usr/bin/env python3
"""Benchmark of the Mamba selective-scan forward path on one MI355X.

One step = the whole hot path over one synthetic batch: depthwise causal conv1d
(width 4) + SiLU, then the selective scan (softplus step sizes, exp(dt A)
discretisation, the recurrence, C.h + D.u readout, SiLU(z) gate, per-document
resets, final state).  Inputs are generated on the host with the seeded recipe
of `workloads`, uploaded once, and are resident in HBM before timing starts.

Prints one JSON line.  `value` is tokens/s of the step (conv + scan; by default
one fused mamba_conv_scan_fwd call).  Extra objects: `roofline` for the timed
call (live HIP-event timing), the HBM roofline of the conv + scan pair, a device
copy probe, and `cpu_baseline` (the fp64 oracle timed on this host on a bounded
sample).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan fwd tokens/s + % HBM roofline, B=2 L=32K D=1536 N=16 bf16"
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0


def scan_bytes(B, L, D, N, nheads, esz):
    """Algorithmic HBM bytes of one selective-scan call: every input read once,
    every output written once (u, delta, z, out, B, C, doc flags, params, state)."""
    nd = nheads if nheads else D
    per_token = esz * (D + nd + D + D) + 2 * esz * N + 1
    params = 4 * ((nheads if nheads else D * N) + D + nd)
    return B * L * per_token + params + B * D * N * 4


def conv_bytes(B, L, D, esz):
    """Algorithmic HBM bytes of one conv call: x read, u written, doc flags, weights."""
    return B * L * (2 * esz * D + 1) + D * 5 * 4


def scan_alu_flop_eq(B, L, D, N, nheads):
    """Algorithmic fp32 VALU work of one scan call in flop-equivalents.

    Counted in full-rate VALU issue slots (an FMA is one slot = 2 flops; a
    transcendental v_exp/v_log/v_rcp runs at quarter rate = 4 slots = 8 flops),
    so that the chip's 157.3 TFLOP/s fp32 vector peak is the matching ceiling.
    Per (t, d, n) element, per-channel A: dt*A (1) + exp (4) + dt*u*B (1) + state
    FMA (1) + C*h FMA (1) = 8 slots.  Scalar-A heads: dt*u*B + two FMAs = 3 slots,
    plus one exp per (t, head).  Per (t, d): softplus (exp + log + 5) = 13, SiLU
    (exp + rcp + 2) = 10, dt*u, D*u, gate = 3 slots (softplus per head for heads)."""
    el = B * L * D * N
    if nheads == 0:
        slots = el * 8 + B * L * D * 26
    else:
        slots = el * 3 + B * L * D * 13 + B * L * nheads * (13 + 4 + 1)
    return 2.0 * slots


def ssd_mfma_flops(B, L, D, N, H, q=64):
    """bf16 MFMA flops the chunked matrix form of scalar-A heads issues per call:
    per 64-token chunk and head, the causal C B^T tiles (10 of the 16 16x16 tiles,
    K = N), M x over the causal K range (K = 32, 32, 64, 64 for the four 16-row
    tiles), C H_in (Q x N x P) and the state update (N x Q x P) in the output pass,
    and the state update again in the aggregate pass."""
    P = D // H
    npad = -(-N // 32) * 32
    per_chunk = (10 * 16 * 16 * npad + 16 * P * (32 + 32 + 64 + 64) + q * npad * P + npad * P * q) * 2
    per_chunk += npad * P * q * 2
    return B * H * (-(-L // q)) * per_chunk


def bwd_bytes(B, L, D, N, esz):
    """Algorithmic HBM bytes of one backward call: u, delta, z, dout, B, C and the
    doc flags read once; du, ddelta, dz, dB, dC written once; parameters and their
    gradients."""
    per_token = esz * 7 * D + 4 * esz * N + 1
    return B * L * per_token + 4 * 2 * (D * N + 3 * D)


def conv_bwd_bytes(B, L, D, esz):
    """Algorithmic HBM bytes of one conv backward call: x and du read, dx written,
    doc flags, weights and their gradients."""
    return B * L * (3 * esz * D + 1) + D * 10 * 4


def bwd_alu_flop_eq(B, L, D, N):
    """Algorithmic fp32 VALU work of the backward in flop-equivalents (slots as in
    scan_alu_flop_eq).  Per (t, d, n): the decay (dt*A + exp = 5), the state
    (dt*u*B, FMA = 2), the adjoint (C*dy FMA, times the decay = 2), a*h_{t-1} and
    g*(a*h) (2), the A and dA terms (2), g.B (1), the dB and dC terms (2) and their
    sums over channels (2) = 18 slots.  Per (t, d): softplus, its sigmoid, SiLU(z)
    with its derivative, du, ddt, dz and the dD / ddelta_bias sums, about 48 slots."""
    return 2.0 * (B * L * D * N * 18 + B * L * D * 48)


def conv_alu_flop_eq(B, L, D):
    """4 FMAs + SiLU (exp, rcp, 2 ops) per (t, d) = 14 slots."""
    return 2.0 * 14 * B * L * D


def copy_probe(torch, dev, mib=1024, reps=5):
    """Device-to-device copy of `mib` MiB (read + write), timed with HIP events on the
    current stream: the measured streaming ceiling the algorithmic GB/s is set against.
    Its kernel also calibrates the FETCH_SIZE / WRITE_SIZE counters in profiling runs."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del src, dst
    return {"bytes_per_copy": 2 * n, "ms": ms, "GBs": 2 * n / (ms * 1e-3) / 1e9}


# The kernel sources each timed path is compiled from: a recorded FETCH/WRITE
# profile counts only while these files are unchanged.
FWD_SOURCES = ["device_common.hpp", "launch.hpp", "conv1d.hip", "scan.hip", "ssd.hip"]
BWD_SOURCES = ["device_common.hpp", "launch.hpp", "scan_bwd.hip", "conv1d_bwd.hip"]


def recorded_traffic(path, source_files):
    """HBM bytes per scan call from the committed FETCH_SIZE / WRITE_SIZE profile, or None
    when the kernel sources have changed since those counters were taken."""
    import hashlib

    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in source_files:
        h.update(open(f, "rb").read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return float(fields["scan_call_hbm_bytes"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, tokens_per_row):
    """Time the fp64 oracle (conv + scan, as it stands) on the first tokens of every row."""
    from threadpoolctl import threadpool_limits

    import oracle

    T = min(tokens_per_row, inp.x.shape[1])
    sl = slice(0, T)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        u = oracle.causal_conv1d(inp.x[:, sl], inp.conv_w, inp.conv_b, inp.doc_start[:, sl])
        oracle.selective_scan(u, inp.delta[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl], inp.D, inp.z[:, sl],
                              inp.delta_bias, True, inp.doc_start[:, sl])
        dt = time.perf_counter() - t0
    ntok = inp.x.shape[0] * T
    return dict(value=ntok / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {T} tokens of each of the {inp.x.shape[0]} rows, all {inp.x.shape[2]} channels "
                       f"({ntok} tokens, {dt:.1f} s, fp64 numpy, one thread)")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="packed_32k",
                    help="workload name from workloads.CONFIGS (default: the 32K packed bf16 shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32768, help="oracle sample: tokens per row")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the device copy probe (0: skip)")
    ap.add_argument("--path", choices=("fused", "split", "bwd", "decode"), default="fused",
                    help="fused: one mamba_conv_scan_fwd call per step; split: conv call, then scan call; "
                         "bwd: scan backward then conv backward (per-channel A workloads); "
                         "decode: one token per row (conv window update + recurrence step)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the scan shards over batch rows and channels with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import selective_state_space_23_amd as ssm
    from workloads import CONFIGS, make_inputs

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_helpers import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ssm._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    spec = CONFIGS[args.config]
    inp = make_inputs(args.config)
    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    H = inp.nheads
    esz = 2 if inp.dtype == "bf16" else 4
    t = upload(inp, dev)
    u = torch.empty_like(t["x"])
    out = torch.empty_like(t["x"])
    fin = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ssm.scan_workspace_bytes(B, L, D, N, H, inp.dtype), 1), dtype=torch.uint8, device=dev)

    if args.path == "bwd":
        return bench_bwd(args, torch, np, ssm, inp, t, spec, dev)
    if args.path == "decode":
        return bench_decode(args, torch, np, ssm, inp, t, spec, dev)
    fused = args.path == "fused"

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if fused:
            ssm.conv_scan_fwd(t["x"], t["conv_w"], t["conv_b"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"], t["doc_start"], u=u, out=out, final_state=fin, workspace=ws)
            if ev is not None:
                ev[1].record()
        else:
            ssm.causal_conv1d_fwd(t["x"], t["conv_w"], t["conv_b"], t["doc_start"], out=u)
            if ev is not None:
                ev[1].record()
            ssm.selective_scan_fwd(u, t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                   t["doc_start"], out=out, final_state=fin, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # HIP events on torch's current stream, which is the stream the binding
    # passes to every launch of the library.
    call_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in events]))
    first_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))

    probe = copy_probe(torch, dev, args.copy_mib) if args.copy_mib > 0 else None
    csrc = os.path.join(ROOT, "selective_state_space_23_amd", "csrc")
    traffic = recorded_traffic(
        os.path.join(ROOT, "profiles", f"{args.path}_{args.config}_hbm_traffic.txt"),
        [os.path.join(csrc, f) for f in FWD_SOURCES])

    tokens = B * L
    sb = scan_bytes(B, L, D, N, H, esz)
    cb = conv_bytes(B, L, D, esz)
    scan_flops = scan_alu_flop_eq(B, L, D, N, H)
    conv_flops = conv_alu_flop_eq(B, L, D)
    if fused:
        kernel = ("mamba_conv_scan_fwd, one call: conv + aggregate pass, carry pass, output pass"
                  if H == 0 else "mamba_conv_scan_fwd, one call: conv, aggregate pass, carry pass, output pass")
        dom_ms, dom_flops, dom_bytes = call_ms, scan_flops + conv_flops, sb + cb
        timings = {"call_ms": call_ms}
    else:
        kernel = "mamba_selective_scan_fwd, one call: aggregate pass, carry pass, output pass"
        dom_ms, dom_flops, dom_bytes = call_ms - first_ms, scan_flops, sb
        timings = {"conv_ms": first_ms, "scan_ms": call_ms - first_ms}
    dom_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    pair_gbs = (sb + cb) / (call_ms * 1e-3) / 1e9
    if H > 0 and inp.dtype == "bf16":
        # Scalar-A heads run as bf16 matrix products: the chunked form's flops go to
        # the matrix cores and the call is measured against HBM (its MFMA share beside).
        mf = ssd_mfma_flops(B, L, D, N, H)
        roof = {"kernel": kernel, "bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dom_gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": dom_bytes,
                "mfma_flops": mf, "mfma_TFLOPs": mf / (dom_ms * 1e-3) / 1e12,
                "mfma_frac": mf / (dom_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, "avg_ms": dom_ms}
    else:
        roof = {"kernel": kernel, "bound": "alu", "achieved": dom_tflops, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": dom_tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic,
                "algorithmic_flop_eq": dom_flops, "algorithmic_bytes": dom_bytes, "hbm_achieved_GBs": dom_gbs,
                "hbm_frac": dom_gbs / HBM_PEAK_GBS, "avg_ms": dom_ms}
    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "batch": B, "seqlen": L, "dim": D, "dstate": N, "nheads": H,
                   "d_conv": 4, "doc_mean_len": spec["docs"], "io_dtype": inp.dtype, "state_dtype": "f32",
                   "path": args.path},
        "roofline": roof,
        "hbm_roofline_pair": dict(
            {"achieved": pair_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pair_gbs / HBM_PEAK_GBS,
             "algorithmic_bytes": sb + cb, "conv_bytes": cb, "scan_bytes": sb}, **timings),
        "copy_probe": None if probe is None else dict(
            probe, pair_frac_of_copy=pair_gbs / probe["GBs"], kernel="hipMemcpyAsync device-to-device"),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(result), flush=True)


METRIC_BWD = "conv + selective-scan bwd tokens/s, B=2 L=32K D=1536 N=16 bf16"


def bench_decode(args, torch, np, ssm, inp, t, spec, dev, tokens=64, graphs_per_run=None):
    """One step = one token for every row: mamba_conv_state_update (the conv
    window update and the recurrence step in one launch) on the workload's rows
    and channels, state and window updated in place.  The timed loop replays a
    HIP graph that holds `tokens` consecutive steps (the steps are launch-bound);
    the eager rate (Python marshalling included) and the two-launch step
    (mamba_causal_conv1d_update, then mamba_selective_state_update) are reported
    beside it."""
    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    H = inp.nheads
    esz = 2 if inp.dtype == "bf16" else 4
    T = min(tokens, L)
    # per-step inputs as (T, B, ...) so every step's slice is contiguous
    xs = t["x"][:, :T].transpose(0, 1).contiguous()
    zs = t["z"][:, :T].transpose(0, 1).contiguous()
    dls = t["delta"][:, :T].transpose(0, 1).contiguous()
    Bs = t["B"][:, :T].transpose(0, 1).contiguous()
    Cs = t["C"][:, :T].transpose(0, 1).contiguous()
    rs = t["doc_start"][:, :T].transpose(0, 1).contiguous()
    rs[0].fill_(1)
    state = torch.zeros((B, D, N), dtype=torch.float32, device=dev)
    cstate = torch.zeros((B, D, 3), dtype=t["x"].dtype, device=dev)
    us = torch.empty((T, B, D), dtype=t["x"].dtype, device=dev)
    outs = torch.empty((T, B, D), dtype=t["x"].dtype, device=dev)

    def steps_two():
        for k in range(T):
            ssm.causal_conv1d_update(xs[k], cstate, t["conv_w"], t["conv_b"], reset=rs[k], out=us[k])
            ssm.selective_state_update(state, us[k], dls[k], t["A"], Bs[k], Cs[k], t["D"], zs[k], t["delta_bias"],
                                       reset=rs[k], out=outs[k])

    def steps():
        for k in range(T):
            ssm.conv_state_update(xs[k], cstate, t["conv_w"], t["conv_b"], state, dls[k], t["A"], Bs[k], Cs[k],
                                  t["D"], zs[k], t["delta_bias"], reset=rs[k], out=outs[k])

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                     # warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        return g

    for _ in range(3):
        steps()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        steps()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / (5 * T)

    # the two-launch step, for comparison
    g2 = graph_of(steps_two)
    for _ in range(args.warmup):
        g2.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(max(args.steps, 1)):
        g2.replay()
    e1.record()
    torch.cuda.synchronize()
    two_us = e0.elapsed_time(e1) * 1e3 / (max(args.steps, 1) * T)

    g = graph_of(steps)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    reps = max(args.steps, 1)
    e0.record()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = e0.elapsed_time(e1) * 1e3 / (reps * T)
    ms_per_step = wall * 1e3 / (reps * T)
    # algorithmic bytes of one step: state and conv window read and written,
    # the token's x, delta, z, B, C read, u and out written, the parameters read
    nd = H if H else D
    nbytes = (2 * B * D * N * 4 + 2 * B * D * 3 * esz + B * (3 * D + nd + 2 * N) * esz + 2 * B * D * esz
              + 4 * ((H if H else D * N) + 2 * D + nd + 4 * D) + B)
    gbs = nbytes / (step_us * 1e-6) / 1e9
    result = {
        "metric": f"selective-scan decode tokens/s, B={B} D={D} N={N} {inp.dtype} (one token per row per step)",
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": reps * T,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "batch": B, "dim": D, "dstate": N, "nheads": H, "io_dtype": inp.dtype,
                   "path": "decode", "tokens_per_graph": T},
        "timings": {"graph_step_us": step_us, "eager_step_us": eager_us, "two_launch_graph_step_us": two_us},
        "roofline": {"kernel": "one decode step: mamba_conv_state_update, one launch (HIP graph replay)",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                     "avg_ms": step_us * 1e-3,
                     "note": "launch-bound: one launch of a few microseconds per token"},
    }
    print(json.dumps(result), flush=True)


def bench_bwd(args, torch, np, ssm, inp, t, spec, dev):
    """One step = the mixer core's backward: mamba_selective_scan_bwd (gradients of
    sum(dout * out) with respect to u, delta, A, B, C, D, z and delta_bias, u being
    the conv output the forward stores) then mamba_causal_conv1d_bwd (dx and the
    conv's weight and bias gradients from du)."""
    from gpu_helpers import to_dev
    from workloads import make_cotangent

    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    if inp.nheads:
        print("the backward pass covers per-channel A workloads only", file=sys.stderr)
        sys.exit(2)
    esz = 2 if inp.dtype == "bf16" else 4
    dout = to_dev(make_cotangent(B, L, D, dtype=inp.dtype, seed=7), inp.dtype, dev)
    ws = torch.empty(ssm.scan_bwd_workspace_bytes(B, L, D, N, inp.dtype), dtype=torch.uint8, device=dev)
    grads = {}

    # u as the forward leaves it (the conv output, stored in the I/O dtype)
    u = ssm.causal_conv1d_fwd(t["x"], t["conv_w"], t["conv_b"], t["doc_start"])
    ws_conv = torch.empty(ssm.conv_bwd_workspace_bytes(B, L, D), dtype=torch.uint8, device=dev)
    conv_grads = {}

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        g = ssm.selective_scan_bwd(u, t["delta"], t["A"], t["B"], t["C"], dout, t["D"], t["z"],
                                   t["delta_bias"], t["doc_start"], workspace=ws, grads=grads)
        grads.update(g)
        if ev is not None:
            ev[1].record()
        dx, dw, db = ssm.causal_conv1d_bwd(t["x"], t["conv_w"], grads["du"], t["conv_b"], t["doc_start"],
                                           workspace=ws_conv, dx=conv_grads.get("dx"),
                                           dweight=conv_grads.get("dw"), dbias=conv_grads.get("db"))
        conv_grads.update(dx=dx, dw=dw, db=db)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    conv_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    probe = copy_probe(torch, dev, args.copy_mib) if args.copy_mib > 0 else None
    csrc = os.path.join(ROOT, "selective_state_space_23_amd", "csrc")
    traffic = recorded_traffic(os.path.join(ROOT, "profiles", f"bwd_{args.config}_hbm_traffic.txt"),
                               [os.path.join(csrc, f) for f in BWD_SOURCES])
    flops = bwd_alu_flop_eq(B, L, D, N)
    nbytes = bwd_bytes(B, L, D, N, esz)
    cbytes = conv_bwd_bytes(B, L, D, esz)
    tflops = flops / (call_ms * 1e-3) / 1e12
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC_BWD,
        "value": B * L / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "batch": B, "seqlen": L, "dim": D, "dstate": N, "nheads": 0,
                   "doc_mean_len": spec["docs"], "io_dtype": inp.dtype, "state_dtype": "f32", "path": "bwd"},
        "timings": {"scan_bwd_ms": call_ms, "conv_bwd_ms": conv_ms,
                    "conv_bwd_hbm_GBs": cbytes / (conv_ms * 1e-3) / 1e9,
                    "conv_bwd_hbm_frac": cbytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"kernel": "mamba_selective_scan_bwd, one call: aggregate pass, forward and reverse carries, "
                               "main pass, reductions",
                     "bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic, "algorithmic_flop_eq": flops,
                     "algorithmic_bytes": nbytes, "hbm_achieved_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "avg_ms": call_ms},
        "copy_probe": probe,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_bwd(inp, dout_seed=7, tokens_per_row=min(args.cpu_tokens, 4096))
    print(json.dumps(result), flush=True)


def cpu_baseline_bwd(inp, dout_seed, tokens_per_row):
    """Time the fp64 oracle gradients (scan, then conv; as they stand) on the first
    tokens of every row."""
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import make_cotangent

    B, L, D = inp.x.shape
    T = min(tokens_per_row, L)
    sl = slice(0, T)
    dout = make_cotangent(B, L, D, dtype=inp.dtype, seed=dout_seed)[:, sl]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        g = oracle.selective_scan_bwd(inp.x[:, sl], inp.delta[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl], dout,
                                      D=inp.D, z=inp.z[:, sl], delta_bias=inp.delta_bias,
                                      doc_start=inp.doc_start[:, sl])
        oracle.causal_conv1d_bwd(inp.x[:, sl], inp.conv_w, g["du"], inp.conv_b, inp.doc_start[:, sl])
        dt = time.perf_counter() - t0
    ntok = B * T
    return dict(value=ntok / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {T} tokens of each of the {B} rows, all {D} channels "
                       f"({ntok} tokens, {dt:.1f} s, fp64 numpy, one thread)")


if __name__ == "__main__":
    main()
