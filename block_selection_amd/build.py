"""Builds libpisa.so (HIP, gfx950) in-tree with hipcc, and libpisa_ceilings.so
(the benchmark's probes of the device ceilings).

Usage: ``python -m block_selection_amd.build``. The libraries land next to
this file, where ``block_selection_amd.ops`` and bench.py load them from.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpisa.so")
SOURCES = ["pyramid.hip", "upper.hip", "leaf.hip", "cluster.hip", "decode.hip", "attention.hip", "flat.hip",
           "api.hip"]
ARCH = os.environ.get("PISA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # inputs are finite by contract (NaN inputs give unspecified indices); lets max/min
    # skip operand canonicalisation. Infinities stay honoured (-inf is a sentinel).
    "-fno-honor-nans",
    # MFMA results in ordinary VGPRs (no accumulation-register copies): fewer registers and
    # VALU moves in the leaf, attention and flat kernels
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


# measurement probes of the device ceilings (not part of the selection), a library of their own
CEILINGS_SOURCES = ["ceilings.hip"]
CEILINGS_LIB = os.path.join(PKG, "libpisa_ceilings.so")


def _compile(sources, out: str, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds libpisa.so and the ceilings probe library; returns the path of libpisa.so."""
    _compile(CEILINGS_SOURCES, CEILINGS_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
