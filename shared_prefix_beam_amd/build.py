"""Build the HIP library libgr_attn.so in-tree (gfx950).

    python -m shared_prefix_beam_amd.build

Kernels and the C-ABI host code are compiled by hipcc for gfx950 only.
Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgr_attn.so")
SOURCES = [os.path.join(CSRC, "gr_attn_kernels.hip"), os.path.join(CSRC, "gr_attn16.hip"),
           os.path.join(CSRC, "gr_noalloc.hip"),
           os.path.join(CSRC, "gr_beam_step.hip"),
           os.path.join(CSRC, "gr_beam_select.hip"), os.path.join(CSRC, "gr_attn_api.cpp")]
# measurement probes (sustained matrix, HBM and exp2 rates), a library of their own
PEAKS_LIB = os.path.join(PKG, "libgr_peaks.so")
PEAKS_SOURCES = [os.path.join(CSRC, "gr_peaks.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile libgr_attn.so and the probe library libgr_peaks.so (always recompiles)."""
    _build_one(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return _build_one(SOURCES, LIB, verbose)


def _build_one(sources, lib, verbose):
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC] + FLAGS + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature: harmless
    noise = ("is not a recognized feature for this target", "reserved registers", "^   ", "^      |")
    err = "\n".join(l for l in res.stderr.splitlines()
                     if not any(n.strip("^") in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
