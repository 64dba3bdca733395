"""Build libmamba_hip.so in-tree with hipcc for gfx950.

Usage: python -m selective_state_space_23_amd.build [--verbose]
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libmamba_hip.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.cpp", "conv1d.hip", "conv1d_bwd.hip", "scan.hip", "scan_bwd.hip", "ssd.hip", "decode.hip", "fill.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled for all device code: hipcc would otherwise
# form v_pk_fma_f32 / v_pk_mul_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def compile_cmd(out_path: str) -> list:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc_path(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-result", "-I", INCLUDE, *DEVICE_FLAGS, "-o", out_path, *srcs]


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (atomically replaced).  Returns the path."""
    fd, tmp = tempfile.mkstemp(prefix=LIB_NAME + ".", suffix=".tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = "is not a recognized feature for this target"
    stderr = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{stderr}")
    if verbose and stderr.strip():
        print(stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
