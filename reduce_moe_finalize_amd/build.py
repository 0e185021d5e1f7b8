"""Build step for the HIP library (gfx950), in-tree.

``python -m reduce_moe_finalize_amd.build`` compiles ``csrc/*.hip`` (the fused
kernels, the split baseline and the bandwidth probe) into
``libfused_boundary.so`` next to this file.  hipcc cross-compiles for gfx950
without a GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "fused_boundary.hip"),
        os.path.join(HERE, "csrc", "split_baseline.hip"),
        os.path.join(HERE, "csrc", "bandwidth_probe.hip"),
        os.path.join(HERE, "csrc", "residency_probe.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfused_boundary.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the residual contract: products rounded to fp32 before they are added
    "-ffp-contract=off",
    # no packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    # Compiler warnings stay visible; the host pass's note that it does not know
    # the device-only packed-fp32 feature is expected and dropped.
    notes = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops' is not a recognized feature" not in ln]
    if notes:
        sys.stderr.write("\n".join(notes) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
