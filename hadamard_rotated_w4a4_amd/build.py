"""Build libw4a4.so in-tree with hipcc for gfx950 (MI355X).

    python -m hadamard_rotated_w4a4_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a4.so")
CEILINGS_LIB = os.path.join(PKG, "libw4a4_ceilings.so")  # measured ceilings for the benchmark
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "w4a4.hip")]
HEADERS = [os.path.join(CSRC, h) for h in ("common.h", "k_prep.h", "k_rotq.h", "k_route.h", "k_dense.h", "k_smallm.h", "k_grouped.h", "k_w16.h")] + [
    os.path.join(ROOT, "include", "w4a4.h")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no silent multiply-add fusion: the quantisers' codes depend on every
    # rounding step; the GEMM epilogue asks for its fused multiply-adds by name
    "-ffp-contract=off",
    # matrix-core results straight into VGPRs: no accvgpr reads in the epilogue
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into libw4a4.so and the ceiling probes into
    libw4a4_ceilings.so (always recompiles)."""
    _compile(LIB, SOURCES, verbose)
    _compile(CEILINGS_LIB, [os.path.join(CSRC, "ceilings.hip")], verbose)
    return LIB


def _compile(lib: str, sources: list, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
