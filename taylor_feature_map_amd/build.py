"""Builds the HIP shared library libbased.so in-tree for gfx950.

Run as `python -m taylor_feature_map_amd.build`; `__graft_entry__.build()` calls `build()`. Each source
is compiled by hipcc in one step (device and host halves together), then hipcc links the objects. The
kernels' compile unit id is fixed (`-cuid`), so the code object does not depend on the directory the
sources sit in. Objects stay in taylor_feature_map_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbased.so")
# A measurement probe kept out of the product library (bench.py --row-probe).
PROBE = "probe_read.hip"
PROBE_LIB = os.path.join(PKG, "libbased_probe.so")
BUILD_DIR = os.path.join(PKG, "_build")
KERNELS = "based_kernels.hip"
API = "based_api.hip"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = [
    f"--offload-arch={ARCH}",
    # MFMA accumulators in ordinary VGPRs: the state is converted to bf16 by VALU every chunk, which
    # would otherwise need an accumulator-register read per element.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Packed fp32 VALU forms are kept out of the device code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Flags of a one-file build (device and host in one hipcc call), also for variants built elsewhere.
FLAGS = [*DEVICE, *COMMON, "-fPIC", "-shared"]


def _start(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, what):
    out, err = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"{what} failed ({proc.returncode}):\n{err}\n{out}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libbased.so next to this file and return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    p = lambda name: os.path.join(BUILD_DIR, name)  # noqa: E731
    kern = _start([HIPCC, *DEVICE, *COMMON, "-cuid=based_kernels", "-fPIC", "-c", os.path.join(CSRC, KERNELS),
                   "-o", p("based_kernels.o")], verbose)
    api = _start([HIPCC, *DEVICE, *COMMON, "-cuid=based_api", "-fPIC", "-c", os.path.join(CSRC, API),
                  "-o", p("based_api.o")], verbose)
    probe = _start([HIPCC, *DEVICE, *COMMON, "-cuid=probe_read", "-fPIC", "-shared", os.path.join(CSRC, PROBE),
                    "-o", PROBE_LIB + ".tmp"], verbose)
    _finish(kern, "kernels compile")
    _finish(api, "api compile")
    _finish(probe, "probe build")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    tmp = LIB + ".tmp"
    _finish(_start([HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", p("based_kernels.o"), p("based_api.o"),
                    "-o", tmp], verbose), "link")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
