"""Build libvn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m virtual_noise_perturbed_amd.build   (or build() from Python).
The library is written next to this file so it travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvn.so")
PROBE = os.path.join(PKG, "vn_probe")
ARCH = "gfx950"

SOURCES = ["vn_kernels.hip", "vn_api.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvn.so)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libvn.so; returns its path."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-shared", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature and says so; harmless
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(out_tmp, LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """The instruction-rate / hash-throughput calibration probe (an executable)."""
    out_tmp = PROBE + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", CSRC, os.path.join(CSRC, "vn_probe.hip"), "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probe ({res.returncode}):\n{errs}")
    os.replace(out_tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(verbose=True))
