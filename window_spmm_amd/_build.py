"""Builds libwindow_spmm.so (host builders + gfx950 kernels + C-ABI) in place."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwindow_spmm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["status.cpp", "formats.cpp", "reorder.cpp"]
HEADERS = ["common.h", "kernels.h", "device.h"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]
# kernels.hip: MFMA accumulators stay in ordinary VGPRs (the unified register
# file of gfx950), which avoids copies around its two-waves-per-SIMD loops.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# bcsr64_pair.hip runs one wave per SIMD with its accumulators in the
# accumulation registers (its A fragments and B ring fill the VGPRs).
HIP_SOURCES = [("kernels.hip", VGPR_FORM), ("bcsr64_pair.hip", []), ("bcsr64_group.hip", []),
               ("api.hip", [])]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wextra"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    if out.strip():
        sys.stderr.write(out + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src, extra in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([HIPCC] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
