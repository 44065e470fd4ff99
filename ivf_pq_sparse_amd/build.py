"""Build libpqhsa.so (HIP, gfx950) in-tree next to this file.

Usage: python -m ivf_pq_sparse_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["pqhsa_host.cpp", "pqhsa_api.hip", "pqhsa_upload.hip", "pqhsa_step.hip", "pqhsa_attn.hip",
           "pqhsa_fused.hip", "pqhsa_append.hip", "pqhsa_reuse.hip"]
LIB_NAME = "libpqhsa.so"
ARCH = "gfx950"

# Packed fp32 ops are disabled for all device code: the compiler still emits
# plain fp32 FMAs, which is what these kernels are written for.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libpqhsa")


def build(verbose: bool = False) -> str:
    """Compile every source (the HIP kernels and the host logic) into
    ivf_pq_sparse_amd/libpqhsa.so; return its path."""
    out = os.path.join(HERE, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(HERE, "csrc", s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
