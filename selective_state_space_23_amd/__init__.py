"""MI355X (gfx950) Mamba selective-scan forward path.

Python binding over libmamba_hip.so: argument marshalling only.  Every step of
the computation runs in the library's HIP kernels; PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing or the tensors are not on a GPU the calls raise.

    u = causal_conv1d_fwd(x, weight, bias, doc_start)                  # (B, L, D)
    out, h = selective_scan_fwd(u, delta, A, B, C, D, z, delta_bias, doc_start)

    # gradients of sum(dout * out) for per-channel A (training), then through the conv
    g = selective_scan_bwd(u, delta, A, B, C, dout, D, z, delta_bias, doc_start)
    dx, dweight, dbias = causal_conv1d_bwd(x, weight, g["du"], bias, doc_start)

    # decode, one token per row, continuing the prefill above
    u_t = causal_conv1d_update(x_t, conv_state, weight, bias)          # (B, D)
    out_t = selective_state_update(h, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias)
    # or both in one launch
    out_t = conv_state_update(x_t, conv_state, weight, bias, h, delta_t, A, B_t, C_t, D, z_t, delta_bias)
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import MambaArgumentError, MambaError, ScanDims  # noqa: F401

__all__ = [
    "causal_conv1d_fwd",
    "selective_scan_fwd",
    "selective_scan_fwd_noalloc",
    "scan_workspace_bytes",
    "conv_scan_fwd",
    "causal_conv1d_update",
    "selective_state_update",
    "conv_state_update",
    "selective_scan_bwd",
    "scan_bwd_workspace_bytes",
    "causal_conv1d_bwd",
    "conv_bwd_workspace_bytes",
    "MambaError",
    "MambaArgumentError",
    "library_path",
    "version",
]


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> str:
    v = _lib.load().mamba_version()
    return f"{v >> 16}.{(v >> 8) & 255}.{v & 255}"


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.MAMBA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return _lib.MAMBA_DTYPE_BF16
    raise MambaArgumentError(_lib.MAMBA_ERR_INVALID_ARGUMENT, f"unsupported activation dtype {t.dtype}")


def _ptr(t, name, device, dtype=None, shape=None) -> Optional[int]:
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _check_device(x):
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device (the library has no CPU path)")
    return x.device


def causal_conv1d_fwd(x, weight, bias=None, doc_start=None, apply_silu: bool = True, out=None, conv_state=None):
    """Depthwise causal conv1d (width 4) + SiLU; see mamba_causal_conv1d_fwd.

    x (B, L, D) float32/bfloat16; weight (D, 4) or (D, 1, 4) float32; bias (D,)
    float32; doc_start (B, L) uint8/bool; conv_state (B, D, 3) of x's dtype: the
    inputs before token 0 (token 0 then starts a document only where doc_start
    says so).  Returns out (B, L, D), x's dtype."""
    torch = _torch()
    dev = _check_device(x)
    if x.dim() != 3:
        raise ValueError("x must be (B, L, D)")
    Bt, L, Dm = x.shape
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[-1])
    W = weight.shape[-1]
    if doc_start is not None and doc_start.dtype == torch.bool:
        doc_start = doc_start.to(torch.uint8)
    if out is None:
        out = torch.empty_like(x)
    st = _lib.load().mamba_causal_conv1d_fwd(
        _ptr(x, "x", dev), _ptr(weight, "weight", dev, torch.float32, (Dm, W)),
        _ptr(bias, "bias", dev, torch.float32, (Dm,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(conv_state, "conv_state", dev, x.dtype, (Bt, Dm, W - 1)),
        _ptr(out, "out", dev, x.dtype, (Bt, L, Dm)), Bt, L, Dm, W, _dtype_code(x), int(bool(apply_silu)),
        _stream(dev))
    _lib.check(st, "mamba_causal_conv1d_fwd")
    return out


def _scan_dims(Bt, L, Dm, N, nheads, dtype_code, softplus) -> ScanDims:
    return ScanDims(batch=Bt, seqlen=L, dim=Dm, dstate=N, nheads=nheads, ngroups=1, dtype=dtype_code,
                    delta_softplus=int(bool(softplus)))


def scan_workspace_bytes(batch, seqlen, dim, dstate, nheads=0, dtype="bf16") -> int:
    code = _lib.MAMBA_DTYPE_BF16 if dtype == "bf16" else _lib.MAMBA_DTYPE_F32
    dims = _scan_dims(batch, seqlen, dim, dstate, nheads, code, True)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().mamba_selective_scan_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)),
               "mamba_selective_scan_workspace_bytes")
    return int(n.value)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, doc_start=None,
                       delta_softplus: bool = True, out=None, final_state=True, workspace=None,
                       initial_state=None):
    """Selective scan forward; see mamba_selective_scan_fwd.

    u, z (B, L, D); delta (B, L, D) with A (D, N), or delta (B, L, H) with A (H,);
    B, C (B, L, N); D (D,), delta_bias (D,) or (H,), float32.  ``final_state``:
    True to allocate and return it, False/None to skip, or a (B, D, N) float32
    tensor to fill.  ``workspace``: optional uint8 device tensor of at least
    scan_workspace_bytes(...) bytes.  ``initial_state``: optional (B, D, N) float32
    state before token 0 (token 0 then resets only where doc_start[:, 0] is set).
    Returns (out, final_state or None)."""
    torch = _torch()
    dev = _check_device(u)
    if u.dim() != 3:
        raise ValueError("u must be (B, L, D)")
    Bt, L, Dm = u.shape
    N = B.shape[-1]
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    code = _dtype_code(u)
    if doc_start is not None and doc_start.dtype == torch.bool:
        doc_start = doc_start.to(torch.uint8)
    if out is None:
        out = torch.empty_like(u)
    if final_state is True:
        final_state = torch.empty((Bt, Dm, N), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    dims = _scan_dims(Bt, L, Dm, N, nheads, code, delta_softplus)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _lib.check(lib.mamba_selective_scan_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)),
               "mamba_selective_scan_workspace_bytes")
    if need.value and workspace is None:
        workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, "workspace", dev, torch.uint8) if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib.mamba_selective_scan_fwd(
        ctypes.byref(dims),
        _ptr(u, "u", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta, "delta", dev, u.dtype, (Bt, L, nd)),
        _ptr(A, "A", dev, torch.float32, (nheads,) if nheads else (Dm, N)),
        _ptr(B, "B", dev, u.dtype, (Bt, L, N)),
        _ptr(C, "C", dev, u.dtype, (Bt, L, N)),
        _ptr(D, "D", dev, torch.float32, (Dm,)),
        _ptr(z, "z", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(initial_state, "initial_state", dev, torch.float32, (Bt, Dm, N)),
        _ptr(out, "out", dev, u.dtype, (Bt, L, Dm)),
        _ptr(final_state, "final_state", dev, torch.float32, (Bt, Dm, N)),
        ws_ptr, ws_bytes, _stream(dev))
    _lib.check(st, "mamba_selective_scan_fwd")
    return out, final_state


def selective_scan_fwd_noalloc(u, delta, A, B, C, out, D=None, z=None, delta_bias=None, doc_start=None,
                               delta_softplus: bool = True, final_state=None, initial_state=None):
    """Selective scan forward with no workspace; see mamba_selective_scan_fwd_noalloc.

    Arguments as selective_scan_fwd; ``out`` (B, L, D) and the optional
    ``final_state`` (B, D, N) float32 are caller-owned tensors the call fills
    (nothing is allocated here or in the library).  Returns (out, final_state)."""
    torch = _torch()
    dev = _check_device(u)
    if u.dim() != 3:
        raise ValueError("u must be (B, L, D)")
    Bt, L, Dm = u.shape
    N = B.shape[-1]
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    if doc_start is not None and doc_start.dtype == torch.bool:
        raise ValueError("doc_start must be uint8 (a bool mask would need a converted copy)")
    dims = _scan_dims(Bt, L, Dm, N, nheads, _dtype_code(u), delta_softplus)
    st = _lib.load().mamba_selective_scan_fwd_noalloc(
        ctypes.byref(dims),
        _ptr(u, "u", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta, "delta", dev, u.dtype, (Bt, L, nd)),
        _ptr(A, "A", dev, torch.float32, (nheads,) if nheads else (Dm, N)),
        _ptr(B, "B", dev, u.dtype, (Bt, L, N)),
        _ptr(C, "C", dev, u.dtype, (Bt, L, N)),
        _ptr(D, "D", dev, torch.float32, (Dm,)),
        _ptr(z, "z", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(initial_state, "initial_state", dev, torch.float32, (Bt, Dm, N)),
        _ptr(out, "out", dev, u.dtype, (Bt, L, Dm)),
        _ptr(final_state, "final_state", dev, torch.float32, (Bt, Dm, N)),
        _stream(dev))
    _lib.check(st, "mamba_selective_scan_fwd_noalloc")
    return out, final_state


def conv_scan_fwd(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None, delta_bias=None, doc_start=None,
                  delta_softplus: bool = True, initial_state=None, conv_state=None, u=True, out=None,
                  final_state=True, workspace=None):
    """Conv1d (width 4) + SiLU and the selective scan in one call; see mamba_conv_scan_fwd.

    Arguments as causal_conv1d_fwd (x, conv_weight, conv_bias, doc_start,
    conv_state) and selective_scan_fwd (the rest).  ``u``: a (B, L, D) tensor that
    receives the conv output, True (allocate one) or None (the conv output is not
    written).  Returns (u or None, out, final_state or None)."""
    torch = _torch()
    dev = _check_device(x)
    if x.dim() != 3:
        raise ValueError("x must be (B, L, D)")
    Bt, L, Dm = x.shape
    N = B.shape[-1]
    if conv_weight.dim() == 3:
        conv_weight = conv_weight.reshape(conv_weight.shape[0], conv_weight.shape[-1])
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    if doc_start is not None and doc_start.dtype == torch.bool:
        doc_start = doc_start.to(torch.uint8)
    if u is True:
        u = torch.empty_like(x)
    elif u is False:
        u = None
    if out is None:
        out = torch.empty_like(x)
    if final_state is True:
        final_state = torch.empty((Bt, Dm, N), dtype=torch.float32, device=dev)
    elif final_state is False:
        final_state = None
    dims = _scan_dims(Bt, L, Dm, N, nheads, _dtype_code(x), delta_softplus)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _lib.check(lib.mamba_selective_scan_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)),
               "mamba_selective_scan_workspace_bytes")
    if need.value and workspace is None:
        workspace = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, "workspace", dev, torch.uint8) if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib.mamba_conv_scan_fwd(
        ctypes.byref(dims),
        _ptr(x, "x", dev, x.dtype, (Bt, L, Dm)),
        _ptr(conv_weight, "conv_weight", dev, torch.float32, (Dm, 4)),
        _ptr(conv_bias, "conv_bias", dev, torch.float32, (Dm,)),
        _ptr(conv_state, "conv_state", dev, x.dtype, (Bt, Dm, 3)),
        _ptr(delta, "delta", dev, x.dtype, (Bt, L, nd)),
        _ptr(A, "A", dev, torch.float32, (nheads,) if nheads else (Dm, N)),
        _ptr(B, "B", dev, x.dtype, (Bt, L, N)),
        _ptr(C, "C", dev, x.dtype, (Bt, L, N)),
        _ptr(D, "D", dev, torch.float32, (Dm,)),
        _ptr(z, "z", dev, x.dtype, (Bt, L, Dm)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(initial_state, "initial_state", dev, torch.float32, (Bt, Dm, N)),
        _ptr(u, "u", dev, x.dtype, (Bt, L, Dm)),
        _ptr(out, "out", dev, x.dtype, (Bt, L, Dm)),
        _ptr(final_state, "final_state", dev, torch.float32, (Bt, Dm, N)),
        ws_ptr, ws_bytes, _stream(dev))
    _lib.check(st, "mamba_conv_scan_fwd")
    return u, out, final_state


def causal_conv1d_update(x, conv_state, weight, bias=None, reset=None, apply_silu: bool = True, out=None):
    """Causal conv1d (width 4) + SiLU for one token per row; see mamba_causal_conv1d_update.

    x (B, D); conv_state (B, D, 3) of x's dtype, updated in place (the last three
    inputs of each channel); weight (D, 4) float32; bias (D,); reset (B,)
    uint8/bool.  Returns out (B, D)."""
    torch = _torch()
    dev = _check_device(x)
    if x.dim() != 2:
        raise ValueError("x must be (B, D)")
    Bt, Dm = x.shape
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[-1])
    W = weight.shape[-1]
    if reset is not None and reset.dtype == torch.bool:
        reset = reset.to(torch.uint8)
    if out is None:
        out = torch.empty_like(x)
    st = _lib.load().mamba_causal_conv1d_update(
        _ptr(x, "x", dev), _ptr(conv_state, "conv_state", dev, x.dtype, (Bt, Dm, W - 1)),
        _ptr(weight, "weight", dev, torch.float32, (Dm, W)), _ptr(bias, "bias", dev, torch.float32, (Dm,)),
        _ptr(reset, "reset", dev, torch.uint8, (Bt,)), _ptr(out, "out", dev, x.dtype, (Bt, Dm)),
        Bt, Dm, W, _dtype_code(x), int(bool(apply_silu)), _stream(dev))
    _lib.check(st, "mamba_causal_conv1d_update")
    return out


def selective_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, reset=None,
                           delta_softplus: bool = True, out=None):
    """One recurrence step per row; see mamba_selective_state_update.

    state (B, D, N) float32, updated in place; u, z (B, D); delta (B, D) with A
    (D, N) or (B, H) with A (H,); B, C (B, N); reset (B,) uint8/bool.  Returns
    out (B, D)."""
    torch = _torch()
    dev = _check_device(u)
    if u.dim() != 2:
        raise ValueError("u must be (B, D)")
    Bt, Dm = u.shape
    N = B.shape[-1]
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    if reset is not None and reset.dtype == torch.bool:
        reset = reset.to(torch.uint8)
    if out is None:
        out = torch.empty_like(u)
    dims = _scan_dims(Bt, 1, Dm, N, nheads, _dtype_code(u), delta_softplus)
    st = _lib.load().mamba_selective_state_update(
        ctypes.byref(dims), _ptr(state, "state", dev, torch.float32, (Bt, Dm, N)),
        _ptr(u, "u", dev, u.dtype, (Bt, Dm)), _ptr(delta, "delta", dev, u.dtype, (Bt, nd)),
        _ptr(A, "A", dev, torch.float32, (nheads,) if nheads else (Dm, N)),
        _ptr(B, "B", dev, u.dtype, (Bt, N)), _ptr(C, "C", dev, u.dtype, (Bt, N)),
        _ptr(D, "D", dev, torch.float32, (Dm,)), _ptr(z, "z", dev, u.dtype, (Bt, Dm)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)), _ptr(reset, "reset", dev, torch.uint8, (Bt,)),
        _ptr(out, "out", dev, u.dtype, (Bt, Dm)), _stream(dev))
    _lib.check(st, "mamba_selective_state_update")
    return out


def scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, dtype="bf16", nheads=0) -> int:
    code = _lib.MAMBA_DTYPE_BF16 if dtype == "bf16" else _lib.MAMBA_DTYPE_F32
    dims = _scan_dims(batch, seqlen, dim, dstate, nheads, code, True)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().mamba_selective_scan_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)),
               "mamba_selective_scan_bwd_workspace_bytes")
    return int(n.value)


def conv_state_update(x, conv_state, conv_weight, conv_bias, state, delta, A, B, C, D=None, z=None, delta_bias=None,
                      reset=None, delta_softplus: bool = True, out=None, u_out=None):
    """Both decode steps in one launch; see mamba_conv_state_update.  x (B, D);
    conv_state (B, D, 3) and state (B, D, N) updated in place; the rest as
    selective_state_update.  Returns out (B, D) (u is written to u_out if given)."""
    torch = _torch()
    dev = _check_device(x)
    if x.dim() != 2:
        raise ValueError("x must be (B, D)")
    Bt, Dm = x.shape
    N = B.shape[-1]
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    if conv_weight.dim() == 3:
        conv_weight = conv_weight.reshape(conv_weight.shape[0], conv_weight.shape[-1])
    if reset is not None and reset.dtype == torch.bool:
        reset = reset.to(torch.uint8)
    if out is None:
        out = torch.empty_like(x)
    dims = _scan_dims(Bt, 1, Dm, N, nheads, _dtype_code(x), delta_softplus)
    st = _lib.load().mamba_conv_state_update(
        ctypes.byref(dims), _ptr(x, "x", dev), _ptr(conv_state, "conv_state", dev, x.dtype, (Bt, Dm, 3)),
        _ptr(conv_weight, "conv_weight", dev, torch.float32, (Dm, 4)),
        _ptr(conv_bias, "conv_bias", dev, torch.float32, (Dm,)),
        _ptr(state, "state", dev, torch.float32, (Bt, Dm, N)), _ptr(delta, "delta", dev, x.dtype, (Bt, nd)),
        _ptr(A, "A", dev, torch.float32, (nheads,) if nheads else (Dm, N)),
        _ptr(B, "B", dev, x.dtype, (Bt, N)), _ptr(C, "C", dev, x.dtype, (Bt, N)),
        _ptr(D, "D", dev, torch.float32, (Dm,)), _ptr(z, "z", dev, x.dtype, (Bt, Dm)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)), _ptr(reset, "reset", dev, torch.uint8, (Bt,)),
        _ptr(u_out, "u_out", dev, x.dtype, (Bt, Dm)), _ptr(out, "out", dev, x.dtype, (Bt, Dm)), _stream(dev))
    _lib.check(st, "mamba_conv_state_update")
    return out


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, doc_start=None,
                       delta_softplus: bool = True, workspace=None, grads=None, initial_state=None,
                       d_final_state=None):
    """Gradients of sum(dout * out) + sum(d_final_state * final_state) for the
    scan; see mamba_selective_scan_bwd.  Arguments as selective_scan_fwd (A
    (D, N) per channel, or (H,) for scalar-A heads with delta (B, L, H)) plus
    ``dout`` (B, L, D) and ``d_final_state`` (B, D, N) float32 or None.  Returns
    a dict with du, ddelta, dB, dC (u's dtype), dA (A's shape) float32 and, for
    each optional input given, dD, dz, ddelta_bias, d_initial_state (B, D, N)
    float32.  ``grads``: optional dict of preallocated outputs with the same
    keys."""
    torch = _torch()
    dev = _check_device(u)
    if u.dim() != 3 or A.dim() not in (1, 2):
        raise ValueError("u must be (B, L, D) and A (D, N) or (H,)")
    Bt, L, Dm = u.shape
    N = B.shape[-1]
    nheads = A.shape[0] if A.dim() == 1 else 0
    nd = nheads if nheads else Dm
    code = _dtype_code(u)
    if doc_start is not None and doc_start.dtype == torch.bool:
        doc_start = doc_start.to(torch.uint8)
    g = dict(grads) if grads else {}
    f32 = torch.float32
    shapes = {"du": ((Bt, L, Dm), u.dtype), "ddelta": ((Bt, L, nd), u.dtype), "dA": (tuple(A.shape), f32),
              "dB": ((Bt, L, N), u.dtype), "dC": ((Bt, L, N), u.dtype)}
    if D is not None:
        shapes["dD"] = ((Dm,), f32)
    if z is not None:
        shapes["dz"] = ((Bt, L, Dm), u.dtype)
    if delta_bias is not None:
        shapes["ddelta_bias"] = ((nd,), f32)
    if initial_state is not None:
        shapes["d_initial_state"] = ((Bt, Dm, N), f32)
    for k, (shape, dt) in shapes.items():
        if k not in g:
            g[k] = torch.empty(shape, dtype=dt, device=dev)
    dims = _scan_dims(Bt, L, Dm, N, nheads, code, delta_softplus)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _lib.check(lib.mamba_selective_scan_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)),
               "mamba_selective_scan_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=dev)
    out = lambda k: _ptr(g.get(k), k, dev, shapes[k][1], shapes[k][0]) if k in shapes else None  # noqa: E731
    st = lib.mamba_selective_scan_bwd(
        ctypes.byref(dims),
        _ptr(u, "u", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta, "delta", dev, u.dtype, (Bt, L, nd)),
        _ptr(A, "A", dev, f32, tuple(A.shape)),
        _ptr(B, "B", dev, u.dtype, (Bt, L, N)),
        _ptr(C, "C", dev, u.dtype, (Bt, L, N)),
        _ptr(D, "D", dev, f32, (Dm,)),
        _ptr(z, "z", dev, u.dtype, (Bt, L, Dm)),
        _ptr(delta_bias, "delta_bias", dev, f32, (nd,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(initial_state, "initial_state", dev, f32, (Bt, Dm, N)),
        _ptr(dout, "dout", dev, u.dtype, (Bt, L, Dm)),
        _ptr(d_final_state, "d_final_state", dev, f32, (Bt, Dm, N)),
        out("du"), out("ddelta"), out("dA"), out("dB"), out("dC"), out("dD"), out("dz"), out("ddelta_bias"),
        out("d_initial_state"),
        _ptr(workspace, "workspace", dev, torch.uint8), workspace.numel(), _stream(dev))
    _lib.check(st, "mamba_selective_scan_bwd")
    return {k: g[k] for k in shapes}


def conv_bwd_workspace_bytes(batch, seqlen, dim) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().mamba_causal_conv1d_bwd_workspace_bytes(batch, seqlen, dim, ctypes.byref(n)),
               "mamba_causal_conv1d_bwd_workspace_bytes")
    return int(n.value)


def causal_conv1d_bwd(x, weight, du, bias=None, doc_start=None, apply_silu: bool = True, workspace=None,
                      dx=None, dweight=None, dbias=None, conv_state=None, d_conv_state=None):
    """Gradients of sum(du * u) for u = causal_conv1d_fwd(x, weight, bias, doc_start,
    conv_state, apply_silu); see mamba_causal_conv1d_bwd.  Returns (dx, dweight
    (D, 4) float32, dbias (D,) float32 or None when bias is None), and with a
    conv_state (B, D, 3) also d_conv_state (B, D, 3) float32 as a fourth item."""
    torch = _torch()
    dev = _check_device(x)
    if x.dim() != 3:
        raise ValueError("x must be (B, L, D)")
    Bt, L, Dm = x.shape
    if weight.dim() == 3:
        weight = weight.reshape(weight.shape[0], weight.shape[-1])
    W = weight.shape[-1]
    if doc_start is not None and doc_start.dtype == torch.bool:
        doc_start = doc_start.to(torch.uint8)
    if dx is None:
        dx = torch.empty_like(x)
    if dweight is None:
        dweight = torch.empty((Dm, W), dtype=torch.float32, device=dev)
    if dbias is None and bias is not None:
        dbias = torch.empty((Dm,), dtype=torch.float32, device=dev)
    if d_conv_state is None and conv_state is not None:
        d_conv_state = torch.empty((Bt, Dm, 3), dtype=torch.float32, device=dev)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _lib.check(lib.mamba_causal_conv1d_bwd_workspace_bytes(Bt, L, Dm, ctypes.byref(need)),
               "mamba_causal_conv1d_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=dev)
    st = lib.mamba_causal_conv1d_bwd(
        _ptr(x, "x", dev), _ptr(weight, "weight", dev, torch.float32, (Dm, W)),
        _ptr(bias, "bias", dev, torch.float32, (Dm,)),
        _ptr(doc_start, "doc_start", dev, torch.uint8, (Bt, L)),
        _ptr(conv_state, "conv_state", dev, x.dtype, (Bt, Dm, 3)),
        _ptr(du, "du", dev, x.dtype, (Bt, L, Dm)), _ptr(dx, "dx", dev, x.dtype, (Bt, L, Dm)),
        _ptr(dweight, "dweight", dev, torch.float32, (Dm, W)), _ptr(dbias, "dbias", dev, torch.float32, (Dm,)),
        _ptr(d_conv_state, "d_conv_state", dev, torch.float32, (Bt, Dm, 3)),
        Bt, L, Dm, W, _dtype_code(x), int(bool(apply_silu)),
        _ptr(workspace, "workspace", dev, torch.uint8), workspace.numel(), _stream(dev))
    _lib.check(st, "mamba_causal_conv1d_bwd")
    if conv_state is not None:
        return dx, dweight, dbias, d_conv_state
    return dx, dweight, dbias
