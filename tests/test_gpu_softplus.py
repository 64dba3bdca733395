"""Accuracy of the kernels' softplus (device_common.hpp, evaluated on the GPU
through the probe library) against the oracle's float64 softplus: the step size
dt = softplus(delta + delta_bias) enters every decay exp(dt A), and the usual
step sizes (1e-3 .. 0.1) come from its far-left tail, where log(1 + e^v)
evaluated naively loses digits."""

import ctypes
import os

import numpy as np
import pytest

import oracle

from gpu_helpers import torch_mod

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "selective_state_space_23_amd",
                     "libmamba_probe.so")


def test_softplus_relative_error():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    assert os.path.exists(PROBE), "libmamba_probe.so is not built"
    lib = ctypes.CDLL(PROBE)
    lib.probe_softplus.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.probe_softplus.restype = ctypes.c_int
    rng = np.random.default_rng(5)
    v = np.concatenate([np.linspace(-30.0, 30.0, 600001), rng.uniform(-8.0, 0.0, 400000),
                        [0.0, -0.0, 1e-30, -1e-30, 88.0, -87.0, -104.0]]).astype(np.float32)
    dv = torch.from_numpy(v).cuda()
    out = torch.empty_like(dv)
    st = lib.probe_softplus(dv.data_ptr(), out.data_ptr(), v.size, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.softplus(v.astype(np.float64))
    rel = np.abs(got - ref) / np.maximum(ref, np.finfo(np.float32).tiny)
    # the usual step-size range: dt in [1e-4, 1] (v in about [-9.2, 0.54])
    usual = (ref >= 1e-4) & (ref <= 1.0)
    print(f"softplus max rel err: all {rel.max():.3g}, dt in [1e-4, 1]: {rel[usual].max():.3g}", flush=True)
    assert rel[usual].max() < 2e-6
    assert rel.max() < 1e-5
