"""Seeded synthetic inputs for the selective-scan path.

This package holds only input recipes (shapes, distributions, document
packing and bf16 rounding of the drawn values).  It contains none of the
method's arithmetic, so both the CPU oracle and the HIP path can be fed from
it without sharing any computation.
"""

from .synth import (  # noqa: F401
    make_cotangent,
    CONFIGS,
    ScanInputs,
    bf16_bits,
    bf16_round,
    config_names,
    make_custom,
    make_inputs,
    pack_documents,
)
