"""Builds libdmr.so (the HIP kernels and the C ABI of include/dmr.h) for gfx950.

    python -m differentiable_mesh_rasterization_amd.build

The library is built in-tree, next to this file, so that it travels with the
source tree. Flags that matter for results:
  -ffp-contract=off      no fused multiply-add: every binary32 operation of the
                         per-pixel evaluation is rounded on its own, in order;
  -munsafe-fp-atomics    float atomicAdd lowers to the hardware float atomic;
  -packed-fp32-ops off   packed FP32 instructions are not generated.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libdmr.so")
SOURCES = ["api.hip", "raster_fwd.hip", "raster_bwd.hip", "blend.hip", "project.hip", "points.hip"]
HEADERS = ["dmr_internal.h", "lds_accum.h", os.path.join("..", "..", "include", "dmr.h")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out_path: str = LIB_PATH, verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source and link libdmr.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
