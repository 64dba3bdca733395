"""Input recipes for the Mamba selective-scan forward path.

Shapes and distributions follow the workloads the pages describe:

* the S6 block of the "Mamba & State Space Models" skill page ("Mamba:
  Selective State Spaces (S6)"): d_conv = 4, A_log initialised to
  log(1..N) so that A = -(n+1), D = ones, tensors laid out (B, L, D);
* the same page's "Key Training Tips": the dt bias is the inverse softplus
  of U(0.001, 0.1);
* the axolotl "FLA Mamba and Mamba2" page: packed rows whose documents each
  start with fresh convolution and recurrent state, and a 32K/64K, hidden
  768 (expand 2 -> 1536 channels), batch 2 BF16 microbenchmark shape;
* the state-spaces/mamba overview: mamba-130m (768 wide) and mamba-2.8b
  (2560 wide) model dimensions; the skill page's "Mamba-2" section:
  d_state 128, headdim 64.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed
order (document lengths, x, z, delta, delta_bias, A noise, B, C, conv
weight).  Values are drawn in float32; for bf16 workloads the activations
(x, z, delta, B, C) are rounded to the nearest bf16 (ties to even) and kept
as float32 arrays holding exactly representable bf16 values.  Parameters
(A, D, delta_bias, conv weight and bias) stay float32.

Nothing here evaluates any step of the method itself.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# ----------------------------------------------------------------------------
# Named workloads.  "docs" is the mean document length of the geometric
# packing, or None for one document per row.
# ----------------------------------------------------------------------------
CONFIGS: Dict[str, dict] = {
    # Tiny single-document fp32 case, small enough for brute force.
    "tiny_f32": dict(batch=1, seqlen=64, dim=16, dstate=4, nheads=0, dtype="f32",
                     docs=None, a_noise=0.0, seed=0),
    # One mamba-130m layer: 768 x expand 2 channels, 2K tokens, 8 rows.
    "m130_2k": dict(batch=8, seqlen=2048, dim=1536, dstate=16, nheads=0, dtype="bf16",
                    docs=512, a_noise=0.1, seed=1),
    # The pages' 32K BF16 microbenchmark shape, packed documents.
    "packed_32k": dict(batch=2, seqlen=32768, dim=1536, dstate=16, nheads=0, dtype="bf16",
                       docs=2048, a_noise=0.1, seed=2),
    # mamba-2.8b width (2560 x 2) at 64K tokens, one document.
    "wide_64k": dict(batch=1, seqlen=65536, dim=5120, dstate=16, nheads=0, dtype="bf16",
                     docs=None, a_noise=0.1, seed=3),
    # Mamba-2 shaped scalar-A heads: 24 heads x headdim 64, d_state 128.
    "heads_32k": dict(batch=2, seqlen=32768, dim=1536, dstate=128, nheads=24, dtype="bf16",
                      docs=2048, a_noise=None, seed=4),
}
_ORDER = ["tiny_f32", "m130_2k", "packed_32k", "wide_64k", "heads_32k"]


def config_names():
    return list(_ORDER)


@dataclasses.dataclass
class ScanInputs:
    """One synthetic batch.  All float arrays are float32 numpy arrays."""

    name: str
    dtype: str              # "f32" or "bf16": storage type of x, z, delta, B, C
    nheads: int             # 0: A is (D, N); >0: A is (H,), delta is (B, L, H)
    x: np.ndarray           # (B, L, D) conv input
    conv_w: np.ndarray      # (D, 4)
    conv_b: np.ndarray      # (D,)
    z: np.ndarray           # (B, L, D) gate input
    delta: np.ndarray       # (B, L, D) or (B, L, H), raw (before bias and softplus)
    delta_bias: np.ndarray  # (D,) or (H,)
    A: np.ndarray           # (D, N) or (H,)
    B: np.ndarray           # (B, L, N)
    C: np.ndarray           # (B, L, N)
    D: np.ndarray           # (D,)
    doc_start: np.ndarray   # (B, L) uint8, 1 at the first token of each document

    @property
    def shape(self):
        b, l, d = self.x.shape
        return dict(batch=b, seqlen=l, dim=d, dstate=self.B.shape[-1], nheads=self.nheads)


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------
def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, ties to even.

    Returns float32 values that are exactly representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The uint16 bf16 encoding of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits expects bf16-representable values; call bf16_round first")
    return (bits >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Document packing
# ----------------------------------------------------------------------------
def pack_documents(rng: np.random.Generator, batch: int, seqlen: int,
                   mean_len: Optional[float]) -> np.ndarray:
    """doc_start flags (B, L) uint8 for rows packed with geometric lengths.

    Lengths follow Geometric(p = 1/mean_len) on {1, 2, ...}; the last document of
    a row is cut at L.  Rows are independent.  Token 0 always starts a document."""
    flags = np.zeros((batch, seqlen), dtype=np.uint8)
    flags[:, 0] = 1
    if mean_len is None or seqlen == 0:
        return flags
    p = 1.0 / float(mean_len)
    for b in range(batch):
        pos = 0
        while True:
            pos += int(rng.geometric(p))
            if pos >= seqlen:
                break
            flags[b, pos] = 1
    return flags


def _normal(rng, shape, scale=1.0):
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def make_custom(batch: int, seqlen: int, dim: int, dstate: int, *, nheads: int = 0,
                dtype: str = "bf16", docs: Optional[float] = None, a_noise: Optional[float] = 0.1,
                seed: int = 0, name: str = "custom") -> ScanInputs:
    """Draw one batch with the given shape using the fixed draw order."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    if nheads and dim % nheads:
        raise ValueError("dim must be a multiple of nheads")
    rng = np.random.default_rng(seed)
    doc_start = pack_documents(rng, batch, seqlen, docs)
    x = _normal(rng, (batch, seqlen, dim))
    z = _normal(rng, (batch, seqlen, dim))
    nd = nheads if nheads else dim
    delta = _normal(rng, (batch, seqlen, nd), 0.1)
    dt0 = rng.uniform(0.001, 0.1, size=nd)
    # inverse softplus of the target step size (float64, then stored as float32)
    delta_bias = np.log(np.expm1(dt0)).astype(np.float32)
    if nheads:
        A = (-np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=nheads))).astype(np.float32)
    else:
        base = -np.arange(1, dstate + 1, dtype=np.float64)[None, :].repeat(dim, axis=0)
        if a_noise:
            base = base * np.exp(a_noise * rng.standard_normal(size=(dim, dstate)))
        A = base.astype(np.float32)
    Bm = _normal(rng, (batch, seqlen, dstate))
    Cm = _normal(rng, (batch, seqlen, dstate))
    conv_w = rng.uniform(-0.5, 0.5, size=(dim, 4)).astype(np.float32)
    conv_b = np.zeros(dim, dtype=np.float32)
    Dv = np.ones(dim, dtype=np.float32)
    if dtype == "bf16":
        x, z, delta, Bm, Cm = (bf16_round(v) for v in (x, z, delta, Bm, Cm))
    return ScanInputs(name=name, dtype=dtype, nheads=nheads, x=x, conv_w=conv_w, conv_b=conv_b,
                      z=z, delta=delta, delta_bias=delta_bias, A=A, B=Bm, C=Cm, D=Dv,
                      doc_start=doc_start)


def make_inputs(config, seed: Optional[int] = None, **overrides) -> ScanInputs:
    """Inputs for a named workload (or its index in ``config_names()``).

    ``overrides`` may replace any shape field (e.g. ``seqlen=4096``) to draw a
    smaller batch with the same recipe."""
    if isinstance(config, int):
        config = _ORDER[config]
    spec = dict(CONFIGS[config])
    spec.update(overrides)
    if seed is not None:
        spec["seed"] = seed
    return make_custom(spec["batch"], spec["seqlen"], spec["dim"], spec["dstate"],
                       nheads=spec["nheads"], dtype=spec["dtype"], docs=spec["docs"],
                       a_noise=spec["a_noise"], seed=spec["seed"], name=config)


def make_cotangent(batch: int, seqlen: int, dim: int, *, dtype: str = "bf16", seed: int = 0,
                   channels=None) -> np.ndarray:
    """A seeded gradient of the loss with respect to the scan output (B, L, D),
    standard normal (bf16-exact for bf16), optionally zero outside `channels`."""
    rng = np.random.default_rng(seed)
    g = _normal(rng, (batch, seqlen, dim))
    if channels is not None:
        keep = np.zeros(dim, dtype=bool)
        keep[np.asarray(channels)] = True
        g[:, :, ~keep] = 0.0
    return bf16_round(g) if dtype == "bf16" else g
