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
SOURCES = [os.path.join(CSRC, "gr_attn_kernels.hip"), os.path.join(CSRC, "gr_beam_step.hip"),
           os.path.join(CSRC, "gr_beam_select.hip"), os.path.join(CSRC, "gr_attn_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source into libgr_attn.so (always recompiles)."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
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
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
