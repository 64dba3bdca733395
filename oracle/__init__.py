"""fp64 CPU oracle for the Mamba selective-scan forward path (and its gradients).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the library and its
Python binding never call it, and there is no CPU fallback anywhere in the
product path.  It shares no code with the HIP kernels.
"""

from .mamba_oracle import (  # noqa: F401
    associative_scan,
    brute_force_scan,
    causal_conv1d,
    conv_kernel_scan,
    doc_segment_start,
    selective_scan,
    sigmoid,
    silu,
    softplus,
    ssd_matrix_scan,
)
from .mamba_grad import causal_conv1d_bwd, selective_scan_bwd  # noqa: F401
