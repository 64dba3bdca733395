#!/usr/bin/env python3
"""Benchmark of the Mamba selective-scan forward path on one MI355X.

One step = the whole hot path over one synthetic batch: depthwise causal conv1d
(width 4) + SiLU, then the selective scan (softplus step sizes, exp(dt A)
discretisation, the recurrence, C.h + D.u readout, SiLU(z) gate, per-document
resets, final state).  Inputs are generated on the host with the seeded recipe
of `workloads`, uploaded once, and are resident in HBM before timing starts.

Prints one JSON line.  `value` is tokens/s of the step (conv + scan; by default
one fused mamba_conv_scan_fwd call).  Extra objects: `roofline` for the timed
call (live HIP-event timing; the metric's own quantity, the HBM roofline of the
conv + scan pair), its ALU fraction beside it (fp32 VALU slots priced with the
measured gfx950 issue rates), a device copy probe, call times with the MALL
flushed before every call (median and min), and `cpu_baseline` (the fp64 oracle
timed on this host: one core, and all cores of the GPU's CPU share).

`--path rates` runs the ALU issue-rate probe instead (libmamba_probe.so).
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
# MI355X fp32 vector peak without packed fp32 (which every device file here is
# built without): 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.
FP32_VECTOR_PEAK_TFLOPS = 78.6
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3
CPU_SHARE = 16          # host cores that go with one GPU on the GPU machines
RATES_FILE = os.path.join(ROOT, "profiles", "alu_rates_gfx950.md")


def trans_slots():
    """Cost of v_exp_f32, v_log_f32, v_rcp_f32 in full-rate fp32 VALU issue slots
    (a v_fma_f32 is 1 slot), from the committed rate table of the probe; 4 (the
    quarter rate of earlier CDNA parts) for any kind the table does not hold."""
    out = {"exp": 4.0, "log": 4.0, "rcp": 4.0, "source": "assumed quarter rate"}
    if os.path.exists(RATES_FILE):
        for line in open(RATES_FILE):
            if line.startswith("slots_") and ":" in line:
                k, v = line.split(":", 1)
                out[k[len("slots_"):].strip()] = float(v)
                out["source"] = "profiles/alu_rates_gfx950.md"
    return out


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


def scan_alu_slots(B, L, D, N, nheads, w):
    """Algorithmic fp32 VALU work of one scan call, in full-rate issue slots
    (an FMA, multiply or add is 1 slot; a transcendental costs w[kind] slots).

    Per (t, d, n) element, per-channel A: dt*A, dt*u*B, the state FMA, the C*h
    FMA (4 slots) and one exp.  Scalar-A heads: dt*u*B and the two FMAs (3
    slots), one exp per (t, head).  Per (t, d): softplus (5 ops, exp, log),
    SiLU(z) (3 ops, exp, rcp), dt*u, D*u and the gate (3 ops); softplus per head
    for heads."""
    el = B * L * D * N
    sp = 5 + w["exp"] + w["log"]
    silu = 3 + w["exp"] + w["rcp"]
    if nheads == 0:
        return el * (4 + w["exp"]) + B * L * D * (sp + silu + 3)
    return el * 3 + B * L * nheads * (sp + w["exp"] + 1) + B * L * D * (silu + 3)


def conv_alu_slots(B, L, D, w):
    """4 FMAs + SiLU (3 ops, exp, rcp) per (t, d)."""
    return B * L * D * (4 + 3 + w["exp"] + w["rcp"])


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


def bwd_bytes(B, L, D, N, esz, nheads=0):
    """Algorithmic HBM bytes of one backward call: u, delta, z, dout, B, C and the
    doc flags read once; du, ddelta, dz, dB, dC written once; parameters (A, D,
    delta_bias) and their gradients.  delta is (B, L, H) for scalar-A heads."""
    nd = nheads if nheads else D
    na = nheads if nheads else D * N
    per_token = esz * (5 * D + 2 * nd + 4 * N) + 1
    return B * L * per_token + 4 * 2 * (na + D + nd)


def heads_bwd_mfma_flops(B, L, D, N, H, q=16):
    """fp32 MFMA flops of the scalar-A heads backward per call, from its 16-token
    chunked form (P = D / H channels per head).  Per chunk: the forward pass's
    state update and reverse aggregate (2 products of Q x N x P); in the main pass
    C H, B dH, dY H^T, x dH^T and C^T dY (5 more of Q x N x P), C B^T, dS B and
    dS^T C (3 of Q x Q x N), and M x, M^T dY, dY x^T (3 of Q x Q x P)."""
    P = D // H
    per_chunk = 2 * (7 * q * N * P + 3 * q * q * N + 3 * q * q * P)
    return B * H * (-(-L // q)) * per_chunk


def conv_bwd_bytes(B, L, D, esz):
    """Algorithmic HBM bytes of one conv backward call: x and du read, dx written,
    doc flags, weights and their gradients."""
    return B * L * (3 * esz * D + 1) + D * 10 * 4


def bwd_alu_slots(B, L, D, N, w):
    """Algorithmic fp32 VALU work of one backward call, in slots as in
    scan_alu_slots.  Per (t, d, n): the decay (dt*A + exp), the state (dt*u*B,
    FMA = 2), the adjoint (C*dy FMA, times the decay = 2), a*h_{t-1} and
    g*(a*h) (2), the A and dA terms (2), g.B (1), the dB and dC terms (2) and
    their sums over channels (2) = 14 slots + exp.  Per (t, d): softplus, its
    sigmoid, SiLU(z) with its derivative, du, ddt, dz and the dD / ddelta_bias
    sums: about 30 ops and 5 transcendentals."""
    return B * L * D * N * (14 + w["exp"]) + B * L * D * (30 + 3 * w["exp"] + w["log"] + w["rcp"])


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
HEADS_BWD_SOURCES = ["device_common.hpp", "launch.hpp", "heads_bwd.hip", "pad.hip"]


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    """Cores of this process's CPU share: the affinity set, capped at the share a
    GPU has on the GPU machines."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, CPU_SHARE))


_SHARD_INP = None     # the workload, inherited by the forked oracle workers


def _oracle_fwd_shard(job):
    """The oracle's conv + scan on one (row, channel range) of the shared workload's
    first T tokens; every (row, channel) chain is independent, so the shards
    together are the whole computation.  Returns the shard's seconds."""
    from threadpoolctl import threadpool_limits

    import oracle

    b, c0, c1, T = job
    inp = _SHARD_INP
    ch, rows, ts = slice(c0, c1), slice(b, b + 1), slice(0, T)
    if inp.nheads:
        P = inp.x.shape[2] // inp.nheads
        hs = slice(c0 // P, c1 // P)
        A, delta, bias = inp.A[hs], inp.delta[rows, ts, hs], inp.delta_bias[hs]
    else:
        A, delta, bias = inp.A[ch], inp.delta[rows, ts, ch], inp.delta_bias[ch]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        u = oracle.causal_conv1d(inp.x[rows, ts, ch], inp.conv_w[ch], inp.conv_b[ch], inp.doc_start[rows, ts])
        oracle.selective_scan(u, delta, A, inp.B[rows, ts], inp.C[rows, ts], inp.D[ch], inp.z[rows, ts, ch], bias,
                              True, inp.doc_start[rows, ts])
        return time.perf_counter() - t0


def cpu_baseline(inp, tokens_one_core, tokens_all_cores):
    """Time the fp64 oracle (conv + scan, as it stands) on this host.

    Two legs: one core on the first `tokens_one_core` tokens of every row, and
    all cores of the CPU share on the first `tokens_all_cores` tokens, sharded
    over independent (row, channel range) pieces in forked worker processes.
    Runs before the GPU is initialised (the workers are forked)."""
    import multiprocessing

    global _SHARD_INP
    _SHARD_INP = inp
    Bt, L, Dm = inp.x.shape
    P = Dm // inp.nheads if inp.nheads else 1
    T1 = min(tokens_one_core, L)
    t1 = sum(_oracle_fwd_shard((b, 0, Dm, T1)) for b in range(Bt))
    one = dict(value=Bt * T1 / t1, unit="tokens/s", cores=1, seconds=t1,
               sample=f"first {T1} tokens of each of the {Bt} rows, all {Dm} channels, one process, one thread")
    ncores = host_cores()
    T = min(tokens_all_cores, L)
    per_row = max(1, ncores // Bt)
    step = -(-Dm // per_row)
    step = -(-step // P) * P                       # whole heads per shard
    jobs = [(b, c0, min(c0 + step, Dm), T) for b in range(Bt) for c0 in range(0, Dm, step)]
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(min(ncores, len(jobs))) as pool:
        pool.map(_oracle_fwd_shard, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    _SHARD_INP = None
    return dict(value=Bt * T / wall, unit="tokens/s", cores=min(ncores, len(jobs)), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"first {T} tokens of each of the {Bt} rows, all {Dm} channels, fp64 numpy, "
                       f"{len(jobs)} (row, channel range) shards over {min(ncores, len(jobs))} worker processes of "
                       f"one thread each, {wall:.1f} s wall",
                one_core=one)


def mall_flusher(torch, dev, mib=768):
    """A fill of `mib` MiB: run between timed calls (outside their events) it
    evicts the previous call's data from the 256 MB MALL and the L2."""
    buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    return lambda: buf.fill_(1)


def bench_rates(args):
    """ALU issue rates of gfx950 from the probe library: wave64 instructions
    retired per SIMD per shader clock, for independent chains (throughput) and one
    dependent chain (latency, cycles per instruction)."""
    import ctypes

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_23_amd", "libmamba_probe.so"))
    lib.probe_alu_rate.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_alu_rate.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    names = ["v_fma_f32", "v_mul_f32", "v_add_f32", "v_exp_f32", "v_log_f32", "v_rcp_f32",
             "1 exp : 1 fma", "1 exp : 3 fma", "1 exp : 5 fma"]
    per_step = {6: (4, 4), 7: (2, 6), 8: (1, 5)}   # (exp, fma) chains of the mixes
    results = []
    for kind, name in enumerate(names):
        for chains in ((8,) if kind < 6 else (sum(per_step[kind]),)) + ((1,) if kind < 6 else ()):
            # throughput: 8 waves on every SIMD; latency: one wave per CU
            blocks, threads = (cus * 8, 256) if chains > 1 else (cus, 64)
            iters = 4096 if chains > 1 else 8192
            out = torch.empty(blocks * threads, dtype=torch.float32, device=dev)
            clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
            stream = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(2):
                st = lib.probe_alu_rate(kind, chains, blocks, threads, iters, out.data_ptr(), clk.data_ptr(), stream)
                if st != 0:
                    raise RuntimeError(f"probe_alu_rate({kind}, {chains}) failed: hip error {st}")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.probe_alu_rate(kind, chains, blocks, threads, iters, out.data_ptr(), clk.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
            ghz = float(np.median(c[:, 0] / c[:, 1]) * 0.1)            # s_memrealtime ticks at 100 MHz
            wave_cycles = float(np.median(c[:, 0]))
            instr_per_wave = iters * 8 * chains
            waves = blocks * threads // 64
            rec = dict(kind=name, chains=chains, ms=ms, clock_GHz=ghz)
            if chains > 1:
                simd = cus * 4
                # wave instructions per SIMD per clock over the kernel's span
                rec["wave_instr_per_simd_clock"] = waves * instr_per_wave / (simd * ms * 1e-3 * ghz * 1e9)
                rec["lane_ops_per_s"] = waves * 64 * instr_per_wave / (ms * 1e-3)
            else:
                rec["latency_cycles"] = wave_cycles / instr_per_wave
            results.append(rec)
            print(json.dumps(rec), flush=True)
    fma = next(r for r in results if r["kind"] == "v_fma_f32" and r["chains"] > 1)["wave_instr_per_simd_clock"]
    slots = {}
    for key, name in (("exp", "v_exp_f32"), ("log", "v_log_f32"), ("rcp", "v_rcp_f32")):
        r = next(r for r in results if r["kind"] == name and r["chains"] > 1)
        slots[key] = fma / r["wave_instr_per_simd_clock"]
    print(json.dumps({"metric": "gfx950 fp32 VALU issue rates", "device": props.name, "cus": cus,
                      "fma_wave_instr_per_simd_clock": fma, "trans_slots": slots, "results": results}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="packed_32k",
                    help="workload name from workloads.CONFIGS (default: the 32K packed bf16 shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32768, help="oracle, one core: tokens per row")
    ap.add_argument("--cpu-tokens-all", type=int, default=32768, help="oracle, all cores: tokens per row")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the device copy probe (0: skip)")
    ap.add_argument("--no-u", action="store_true",
                    help="fused path: the conv output u is not written (u = NULL; the output pass forms it again)")
    ap.add_argument("--flush-reps", type=int, default=20,
                    help="calls timed one by one with the MALL flushed before each (0: skip)")
    ap.add_argument("--path", choices=("fused", "split", "bwd", "decode", "rates"), default="fused",
                    help="fused: one mamba_conv_scan_fwd call per step; split: conv call, then scan call; "
                         "bwd: scan backward then conv backward; "
                         "decode: one token per row (conv window update + recurrence step); "
                         "rates: the ALU issue-rate probe")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the scan shards over batch rows and channels with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.path == "rates":
        return bench_rates(args)

    import numpy as np

    from workloads import CONFIGS, make_inputs

    spec = CONFIGS[args.config]
    inp = make_inputs(args.config)
    # The oracle legs run first: their workers are forked before the GPU is touched.
    cpu = None
    if not args.no_cpu_baseline and args.path in ("fused", "split"):
        cpu = cpu_baseline(inp, args.cpu_tokens, args.cpu_tokens_all)
    if not args.no_cpu_baseline and args.path == "bwd":
        # about 10 s of one core (the heads workload, N = 128, costs 4x per token)
        cpu = cpu_baseline_bwd(inp, dout_seed=7, tokens_per_row=min(args.cpu_tokens, 4096 if inp.nheads else 16384))

    import torch

    import selective_state_space_23_amd as ssm
    from workloads.device import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ssm._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    H = inp.nheads
    esz = 2 if inp.dtype == "bf16" else 4
    t = upload(inp, dev)
    if args.path == "bwd":
        return bench_bwd(args, torch, np, ssm, inp, t, spec, dev, cpu)
    if args.path == "decode":
        return bench_decode(args, torch, np, ssm, inp, t, spec, dev)
    u = torch.empty_like(t["x"])
    out = torch.empty_like(t["x"])
    fin = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    if args.no_u and args.path != "fused":
        print("--no-u applies to the fused path", file=sys.stderr)
        sys.exit(2)
    u_arg = None if args.no_u else u
    ws = torch.empty(max(ssm.scan_workspace_bytes(B, L, D, N, H, inp.dtype), 1), dtype=torch.uint8, device=dev)
    fused = args.path == "fused"

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if fused:
            ssm.conv_scan_fwd(t["x"], t["conv_w"], t["conv_b"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                              t["delta_bias"], t["doc_start"], u=u_arg, out=out, final_state=fin, workspace=ws)
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
    call_all = np.array([e[0].elapsed_time(e[2]) for e in events])
    first_all = np.array([e[0].elapsed_time(e[1]) for e in events])
    call_ms, first_ms = float(call_all.mean()), float(first_all.mean())

    # The same call timed one by one with the MALL and L2 flushed before each.
    flushed = None
    if args.flush_reps > 0:
        flush = mall_flusher(torch, dev)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.flush_reps)]
        for e in fev:
            flush()
            e[0].record()
            step()
            e[1].record()
        torch.cuda.synchronize()
        f = np.array([e[0].elapsed_time(e[1]) for e in fev])
        flushed = {"reps": args.flush_reps, "flush_MiB": 768, "call_ms_median": float(np.median(f)),
                   "call_ms_min": float(f.min())}
        del flush

    probe = copy_probe(torch, dev, args.copy_mib) if args.copy_mib > 0 else None
    csrc = os.path.join(ROOT, "selective_state_space_23_amd", "csrc")
    traffic = recorded_traffic(
        os.path.join(ROOT, "profiles", f"{args.path}{'_no_u' if args.no_u else ''}_{args.config}_hbm_traffic.txt"),
        [os.path.join(csrc, f) for f in FWD_SOURCES])

    w = trans_slots()
    tokens = B * L
    sb = scan_bytes(B, L, D, N, H, esz)
    cb = conv_bytes(B, L, D, esz)
    if fused:
        kernel = ("mamba_conv_scan_fwd, one call: conv + aggregate pass, carry pass, output pass"
                  if H == 0 else "mamba_conv_scan_fwd, one call: conv, aggregate pass, carry pass, output pass")
        dom_ms, dom_bytes = call_ms, sb + cb
        dom_slots = scan_alu_slots(B, L, D, N, H, w) + conv_alu_slots(B, L, D, w)
        timings = {"call_ms": call_ms, "call_ms_median": float(np.median(call_all)), "call_ms_min": float(call_all.min())}
    else:
        kernel = "mamba_selective_scan_fwd, one call: aggregate pass, carry pass, output pass"
        dom_ms, dom_bytes = call_ms - first_ms, sb
        dom_slots = scan_alu_slots(B, L, D, N, H, w)
        timings = {"conv_ms": first_ms, "scan_ms": call_ms - first_ms}
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    pair_gbs = (sb + cb) / (call_ms * 1e-3) / 1e9
    # flop-equivalents: a slot is one lane FMA = 2 flops
    alu_tflops = 2.0 * dom_slots / (dom_ms * 1e-3) / 1e12
    roof = {"kernel": kernel, "bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dom_gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": dom_bytes, "avg_ms": dom_ms}
    if H > 0 and inp.dtype == "bf16":
        # Scalar-A heads run as bf16 matrix products: their share of the matrix cores beside.
        mf = ssd_mfma_flops(B, L, D, N, H)
        roof.update(mfma_flops=mf, mfma_TFLOPs=mf / (dom_ms * 1e-3) / 1e12,
                    mfma_frac=mf / (dom_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS)
    else:
        roof["alu"] = {"algorithmic_slots": dom_slots, "achieved_TFLOPs": alu_tflops,
                       "peak_TFLOPs": FP32_VECTOR_PEAK_TFLOPS, "frac": alu_tflops / FP32_VECTOR_PEAK_TFLOPS,
                       "trans_slots": w,
                       "note": "fp32 VALU issue slots of the method's own work (one exp and four fp32 ops per "
                               "(t,d,n), the per-token softplus, SiLU and conv) at the non-packed fp32 peak; "
                               "transcendentals priced at the measured gfx950 rates"}
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
                   "path": args.path, "u_written": not args.no_u},
        "roofline": roof,
        "hbm_roofline_pair": dict(
            {"achieved": pair_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pair_gbs / HBM_PEAK_GBS,
             "algorithmic_bytes": sb + cb, "conv_bytes": cb, "scan_bytes": sb}, **timings),
        "mall_flushed": flushed,
        "copy_probe": None if probe is None else dict(
            probe, pair_frac_of_copy=pair_gbs / probe["GBs"], kernel="hipMemcpyAsync device-to-device"),
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


METRIC_BWD = "conv + selective-scan bwd tokens/s"


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


def bench_bwd(args, torch, np, ssm, inp, t, spec, dev, cpu=None):
    """One step = the mixer core's backward: mamba_selective_scan_bwd (gradients of
    sum(dout * out) with respect to u, delta, A, B, C, D, z and delta_bias, u being
    the conv output the forward stores) then mamba_causal_conv1d_bwd (dx and the
    conv's weight and bias gradients from du)."""
    from workloads.device import to_dev
    from workloads import make_cotangent

    B, L, D = inp.x.shape
    N = inp.B.shape[-1]
    H = inp.nheads
    esz = 2 if inp.dtype == "bf16" else 4
    dout = to_dev(make_cotangent(B, L, D, dtype=inp.dtype, seed=7), inp.dtype, dev)
    ws = torch.empty(ssm.scan_bwd_workspace_bytes(B, L, D, N, inp.dtype, nheads=H), dtype=torch.uint8,
                     device=dev)
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
                               [os.path.join(csrc, f) for f in (HEADS_BWD_SOURCES if H else BWD_SOURCES)])
    nbytes = bwd_bytes(B, L, D, N, esz, H)
    cbytes = conv_bwd_bytes(B, L, D, esz)
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    if H:
        # products of the chunked form on v_mfma_f32_16x16x4f32: the fp32 matrix peak
        flops = heads_bwd_mfma_flops(B, L, D, N, H)
        tflops = flops / (call_ms * 1e-3) / 1e12
        roofline = {"kernel": "mamba_selective_scan_bwd (scalar-A heads), one call: forward pass, carries, "
                              "main pass, reductions",
                    "bound": "mfma", "achieved": tflops, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tflops / FP32_MFMA_PEAK_TFLOPS, "traffic": traffic, "mfma_dtype": "f32",
                    "algorithmic_flops": flops}
    else:
        flops = 2.0 * bwd_alu_slots(B, L, D, N, trans_slots())
        tflops = flops / (call_ms * 1e-3) / 1e12
        roofline = {"kernel": "mamba_selective_scan_bwd, one call: aggregate pass, forward and reverse carries, "
                              "main pass, reductions",
                    "bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic, "algorithmic_flop_eq": flops}
    roofline.update(algorithmic_bytes=nbytes, hbm_achieved_GBs=gbs, hbm_frac=gbs / HBM_PEAK_GBS, avg_ms=call_ms)
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
        "config": {"workload": args.config, "batch": B, "seqlen": L, "dim": D, "dstate": N, "nheads": H,
                   "doc_mean_len": spec["docs"], "io_dtype": inp.dtype, "state_dtype": "f32", "path": "bwd"},
        "timings": {"scan_bwd_ms": call_ms, "conv_bwd_ms": conv_ms,
                    "conv_bwd_hbm_GBs": cbytes / (conv_ms * 1e-3) / 1e9,
                    "conv_bwd_hbm_frac": cbytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": roofline,
        "copy_probe": probe,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
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
