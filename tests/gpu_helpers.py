"""Shared helpers for the GPU parity tests (uploading synthetic inputs, running the
HIP path through the C ABI, running the oracle on the same inputs, comparing).

The oracle side never consumes anything the HIP path produced."""

from __future__ import annotations

import numpy as np

import oracle
from workloads import bf16_round
from workloads.device import to_dev, to_host, upload  # noqa: F401

# Tolerances stated for the path: fp32 I/O to 1e-4 relative; bf16 I/O with fp32
# state to 2e-2 relative / absolute.  fp32 uses an absolute floor of 1e-4 x the
# reference's rms so that entries near zero are measured on the output's scale.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}


def torch_mod():
    import torch
    return torch


def assert_close(got, ref, dtype, what, rms_floor=True):
    rtol, atol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32" and rms_floor:
        atol = atol * max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    err = np.abs(got - ref)
    bad = err > rtol * np.abs(ref) + atol
    if bad.any():
        i = np.unravel_index(np.argmax(err - rtol * np.abs(ref)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance "
                             f"(rtol={rtol}, atol={atol:.3g}); worst at {i}: got {got[i]!r} ref {ref[i]!r}; "
                             f"max abs err {err.max():.3g}")
    return float(err.max())


def per_channel_params(inp, channels):
    """Oracle parameters for a subset of channels, in per-channel (diagonal) form.

    For scalar-A heads, channel d uses its head's A (repeated over the states),
    step size and bias; the oracle's tests pin that this equals the heads form."""
    channels = np.asarray(channels)
    N = inp.B.shape[-1]
    if inp.nheads:
        P = inp.x.shape[2] // inp.nheads
        heads = channels // P
        A = np.repeat(inp.A[heads][:, None], N, axis=1)
        delta = inp.delta[:, :, heads]
        bias = inp.delta_bias[heads]
    else:
        A = inp.A[channels]
        delta = inp.delta[:, :, channels]
        bias = inp.delta_bias[channels]
    return A, delta, bias


def oracle_pipeline(inp, channels, round_u=True, use_z=True, use_D=True, use_bias=True, softplus=True):
    """Oracle conv -> (bf16 boundary rounding of u) -> scan on the given channels."""
    ch = np.asarray(channels)
    u = oracle.causal_conv1d(inp.x[:, :, ch], inp.conv_w[ch], inp.conv_b[ch], inp.doc_start)
    if round_u and inp.dtype == "bf16":
        u = bf16_round(u.astype(np.float32)).astype(np.float64)
    A, delta, bias = per_channel_params(inp, ch)
    out, fin = oracle.selective_scan(u, delta, A, inp.B, inp.C, inp.D[ch] if use_D else None,
                                     inp.z[:, :, ch] if use_z else None, bias if use_bias else None,
                                     softplus, inp.doc_start)
    return u, out, fin


def oracle_scan(inp, u, channels, **kw):
    """Oracle scan alone on given u (B, L, len(channels)) for the given channels."""
    ch = np.asarray(channels)
    A, delta, bias = per_channel_params(inp, ch)
    use_z = kw.pop("use_z", True)
    use_D = kw.pop("use_D", True)
    use_bias = kw.pop("use_bias", True)
    softplus = kw.pop("softplus", True)
    init = kw.pop("initial_state", None)
    return oracle.selective_scan(u, delta, A, inp.B, inp.C, inp.D[ch] if use_D else None,
                                 inp.z[:, :, ch] if use_z else None, bias if use_bias else None, softplus,
                                 inp.doc_start, initial_state=None if init is None else init[:, ch, :])
