"""Build libce.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python vocab_cross_entropy_amd/csrc/build.py [--phases]

--phases builds libce_phases.so instead: the same library with phase stamps
compiled into the fused and statistics kernels (bench.py --phases).

Objects go to _build/ at the repository root; the shared library lands next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

CSRC = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(CSRC)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libce.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
COMMON = ["-std=c++17", "-fPIC", "-O3", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]
# Packed FP32 VALU forms are kept out of the device code.  Multiplies and
# adds are fused only within one expression (-ffp-contract=on; hipcc's default
# fuses across statements): the kernels round m log2(e) once and rely on that
# rounded value wherever it is reused, so that the rounding cancels between the
# sum's terms and its rescaling; a product fused into a later subtraction
# unrounded breaks that.  The fused multiply-adds the kernels want are written
# out as __builtin_fmaf.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=on"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# The instrumented variant: the same sources with the phase stamps compiled in
# (CE_PHASE_CLOCK), for `bench.py --phases`; never loaded by default.
PHASES_LIB = os.path.join(PKG, "libce_phases.so")


def build(verbose: bool = False, variant: str = "") -> str:
    """Build libce.so, or with variant="phases" the instrumented libce_phases.so."""
    if variant not in ("", "phases"):
        raise ValueError(f"unknown variant {variant!r}")
    bdir = os.path.join(BUILD, variant) if variant else BUILD
    lib = PHASES_LIB if variant else LIB
    extra = ["-DCE_PHASE_CLOCK"] if variant else []
    os.makedirs(bdir, exist_ok=True)
    kobj = os.path.join(bdir, "ce_kernels.o")
    aobj = os.path.join(bdir, "ce_api.o")
    lobj = os.path.join(bdir, "ce_linear.o")
    gobj = os.path.join(bdir, "ce_gemm.o")
    robj = os.path.join(bdir, "ce_stream_ref.o")
    steps = [
        [HIPCC, *DEVICE, *COMMON, *extra, "-c", os.path.join(CSRC, "ce_kernels.hip"), "-o", kobj],
        [HIPCC, *DEVICE, *COMMON, *extra, "-c", os.path.join(CSRC, "ce_gemm.hip"), "-o", gobj],
        [HIPCC, *DEVICE, *COMMON, *extra, "-c", os.path.join(CSRC, "ce_stream_ref.hip"), "-o", robj],
        [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, "ce_api.cpp"), "-o", aobj],
        [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, "ce_linear.cpp"), "-o", lobj],
    ]
    for cmd in steps:
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
    tmp = lib + ".tmp"
    # the chunked linear call's products run on the library's MFMA kernel (ce_gemm.hip) or on hipBLASLt
    # (ROCm's matrix-core GEMM library), per ce_linear.gemm
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", kobj, gobj, robj, aobj, lobj, "-L/opt/rocm/lib",
          "-lhipblaslt", "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, variant="phases" if "--phases" in sys.argv else ""))
