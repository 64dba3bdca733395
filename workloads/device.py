"""Moving the synthetic inputs onto a GPU as torch tensors (storage conversion
only: float32 or bf16 bit patterns; no step of the method).  Imported by the
benchmark and the GPU tests; needs torch."""

from __future__ import annotations

import numpy as np

from .synth import bf16_bits


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    """Upload a float32 numpy array as float32 or bf16 (values already bf16-exact)."""
    import torch

    if dtype == "bf16":
        bits = bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t) -> np.ndarray:
    """A device tensor as a float64 numpy array."""
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def upload(inp, device="cuda"):
    """Every array of a ScanInputs on `device`: activations in the workload's
    storage dtype, parameters float32, doc_start uint8."""
    import torch

    dt = inp.dtype
    return dict(
        x=to_dev(inp.x, dt, device), z=to_dev(inp.z, dt, device), delta=to_dev(inp.delta, dt, device),
        B=to_dev(inp.B, dt, device), C=to_dev(inp.C, dt, device),
        conv_w=torch.from_numpy(inp.conv_w).to(device), conv_b=torch.from_numpy(inp.conv_b).to(device),
        A=torch.from_numpy(inp.A).to(device), D=torch.from_numpy(inp.D).to(device),
        delta_bias=torch.from_numpy(inp.delta_bias).to(device),
        doc_start=torch.from_numpy(inp.doc_start).to(device))
