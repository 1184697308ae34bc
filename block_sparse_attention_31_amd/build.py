"""Builds libvdn_local_attn.so in-tree with hipcc for gfx950.

Usage: python -m block_sparse_attention_31_amd.build  (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libvdn_local_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["api.cpp", "schedule.cpp", "fwd_kernel.hip", "fwd_fp8_kernel.hip", "bwd_kernel.hip", "linear_kernel.hip"]

# Packed fp32 VALU instructions are disabled for all device code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN operands reach the kernels' min/max: skip NaN canonicalisation
    "-Xarch_device", "-fno-honor-nans",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so: drop it.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
