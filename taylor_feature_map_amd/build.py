"""Builds the HIP shared library libbased.so in-tree for gfx950 with hipcc.

Run as `python -m taylor_feature_map_amd.build`; `__graft_entry__.build()` calls `build()`.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbased.so")
SOURCES = ["based_kernels.hip", "based_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # MFMA accumulators in ordinary VGPRs: the state is converted to bf16 by VALU every chunk, which
    # would otherwise need an accumulator-register read per element.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Packed fp32 VALU forms are kept out of the device code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libbased.so next to this file and return its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
