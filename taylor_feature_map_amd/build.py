"""Builds the HIP shared library libbased.so in-tree for gfx950.

Run as `python -m taylor_feature_map_amd.build`; `__graft_entry__.build()` calls `build()`.

The device code goes through assembly so that `hazard_pad` can put wait states after wide stores before
it is assembled:
- hipcc --cuda-device-only -S based_kernels.hip gives the gfx950 assembly;
- hazard_pad.pad(); the build then checks that only s_nop lines were added and that the rule holds;
- the LLVM assembler and lld give the code object, clang-offload-bundler wraps it as a HIP fat binary;
- the host half of based_kernels.hip is compiled with that fat binary embedded (the kernel stubs
  register it at load time exactly as in a one-step hipcc build), based_api.hip is compiled as usual,
  and hipcc links both into libbased.so.
Intermediate files stay in taylor_feature_map_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import hazard_pad

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbased.so")
BUILD_DIR = os.path.join(PKG, "_build")
KERNELS = "based_kernels.hip"
API = "based_api.hip"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/lib/llvm/bin")
ARCH = "gfx950"
BUNDLE_TARGETS = f"host-x86_64-unknown-linux-gnu,hipv4-amdgcn-amd-amdhsa--{ARCH}"

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
# One-step flags (device and host in one hipcc call), for builds of variants outside this module.
FLAGS = [*DEVICE, *COMMON, "-fPIC", "-shared"]


def _start(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, what):
    out, err = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"{what} failed ({proc.returncode}):\n{err}\n{out}")


def _run(cmd, what, verbose):
    _finish(_start(cmd, verbose), what)


def device_assembly(out_path: str, verbose: bool = False) -> str:
    """Compile the kernels' device half to gfx950 assembly at `out_path`."""
    _run([HIPCC, "--cuda-device-only", "-S", *DEVICE, *COMMON, os.path.join(CSRC, KERNELS), "-o", out_path],
         "device compile", verbose)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libbased.so next to this file and return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    p = lambda name: os.path.join(BUILD_DIR, name)  # noqa: E731
    # The host halves do not depend on the device code object except through the fat binary, which
    # the kernels' host compile needs, so based_api.hip compiles while the device half does.
    api = _start([HIPCC, *DEVICE, *COMMON, "-fPIC", "-c", os.path.join(CSRC, API), "-o", p("based_api.o")],
                 verbose)
    device_assembly(p("based_kernels.s"), verbose)
    with open(p("based_kernels.s")) as f:
        src = f.read()
    rep = hazard_pad.pad(src)
    padded = "\n".join(rep.lines)
    if not hazard_pad.same_program(src, padded):
        raise RuntimeError("store padding changed more than the added s_nop lines")
    bad = hazard_pad.check(padded)
    if bad:
        raise RuntimeError("store padding left violations:\n" + "\n".join(bad[:20]))
    with open(p("based_kernels.pad.s"), "w") as f:
        f.write(padded)
    if verbose:
        print(f"hazard_pad: {rep.sites} sites, {rep.drains} drains, {rep.waits_added} wait states added",
              flush=True)
    _run([os.path.join(LLVM_BIN, "clang"), "-target", "amdgcn-amd-amdhsa", f"-mcpu={ARCH}", "-c",
          p("based_kernels.pad.s"), "-o", p("based_kernels.dev.o")], "assemble", verbose)
    _run([os.path.join(LLVM_BIN, "ld.lld"), "-flavor", "gnu", "-m", "elf64_amdgpu", "--no-undefined",
          "-shared", p("based_kernels.dev.o"), "-o", p("based_kernels.hsaco")], "device link", verbose)
    _run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "-type=o", "-bundle-align=4096",
          f"-targets={BUNDLE_TARGETS}", "-input=/dev/null", f"-input={p('based_kernels.hsaco')}",
          f"-output={p('based_kernels.hipfb')}"], "bundle", verbose)
    _run([HIPCC, "--cuda-host-only", *DEVICE, *COMMON, "-fPIC", "-Xclang", "-fcuda-include-gpubinary",
          "-Xclang", p("based_kernels.hipfb"), "-c", os.path.join(CSRC, KERNELS), "-o", p("based_kernels.o")],
         "host compile", verbose)
    _finish(api, "api compile")
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", p("based_kernels.o"), p("based_api.o"),
          "-o", tmp], "link", verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
