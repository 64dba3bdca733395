"""Build libmamba_hip.so in-tree with hipcc for gfx950.

Each source is compiled to an object in parallel, then the objects are linked
into one shared library (atomically replacing the previous one).

Usage: python -m selective_state_space_23_amd.build [--verbose]
"""

from __future__ import annotations

import concurrent.futures
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
SOURCES = ["api.cpp", "noalloc.hip", "conv1d.hip", "conv1d_bwd.hip", "scan.hip", "scan_bwd.hip", "ssd.hip",
           "decode.hip", "fill.hip", "pad.hip", "heads_bwd.hip"]
# The ALU issue-rate probe bench.py runs (measurement only, not part of the C ABI).
PROBE_SRC = os.path.join(PKG_DIR, "probe", "alu_rates.hip")
PROBE_PATH = os.path.join(PKG_DIR, "libmamba_probe.so")
ARCH = "gfx950"

# Packed fp32 instructions are disabled for all device code: hipcc would otherwise
# form v_pk_fma_f32 / v_pk_mul_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
_NOISE = "is not a recognized feature for this target"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def compile_cmd(src: str, obj: str) -> list:
    return [hipcc_path(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-c", "-Wall",
            "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, "-o", obj, src]


def link_cmd(objs: list, out_path: str) -> list:
    return [hipcc_path(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_path, *objs]


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    stderr = "\n".join(l for l in proc.stderr.splitlines() if _NOISE not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}\n{stderr}")
    if verbose and stderr.strip():
        print(stderr, file=sys.stderr)


def _link(objs: list, lib_path: str, verbose: bool) -> None:
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(lib_path) + ".", suffix=".tmp", dir=PKG_DIR)
    os.close(fd)
    try:
        _run(link_cmd(objs, tmp), verbose)
    except Exception:
        os.unlink(tmp)
        raise
    os.replace(tmp, lib_path)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source into LIB_PATH and the ALU-rate probe into PROBE_PATH
    (each atomically replaced).  Returns LIB_PATH."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [PROBE_SRC]
    jobs = jobs or min(len(srcs), max(1, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="mamba_hip_build.") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            futs = [pool.submit(_run, compile_cmd(s, o), verbose) for s, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        _link(objs[:-1], LIB_PATH, verbose)
        _link(objs[-1:], PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
