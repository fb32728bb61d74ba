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

SOURCES = ["vn_kernels.hip", "vn_gemm.hip", "vn_api.cpp"]

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


# the compiler's per-kernel resource report (registers, scratch, occupancy)
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def kernels_with_scratch(remarks: str) -> dict:
    """Kernel name -> scratch bytes per lane, for every kernel whose resource
    report (the compiler's kernel-resource-usage remarks) shows scratch."""
    import re
    found, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            found[name] = int(m.group(1))
    return found


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libvn.so; returns its path.  Fails when
    any kernel spills to scratch memory (per-lane stack traffic in the hot
    loops is never intended here)."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, RESOURCE_REMARKS, *(extra_flags or []), "-shared", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature and says so; harmless
    lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n" + "\n".join(lines))
    # (the resource remarks come with source excerpts; only real diagnostics are shown)
    diags = "\n".join(l for l in lines if ("warning:" in l or "error:" in l) and "kernel-resource-usage" not in l)
    if verbose and diags.strip():
        print(diags, file=sys.stderr)
    spills = kernels_with_scratch(res.stderr)
    if spills:
        os.remove(out_tmp)
        raise RuntimeError("kernels use scratch memory (register spills): " +
                           ", ".join(f"{k} ({v} B/lane)" for k, v in sorted(spills.items())))
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
