"""Builds libgsr.so (the HIP kernels and the C ABI of include/gsr.h) in-tree for gfx950.

    python -m differentiable_gaussian_splatting_amd.build

Flags that matter for results:
  -ffp-contract=off      no fused multiply-add contraction: sigma, alpha, T, the colour sums, the tile extents and
                         the Adam update round once per operation, in source order;
  -munsafe-fp-atomics    hardware float atomics (global_atomic_add_f32) for the backward's gradient sums;
  -packed-fp32-ops off   no v_pk_*_f32 packed fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgsr.so")
SOURCES = ["ctx.hip", "bin.hip", "sort.hip", "raster_fwd.hip", "raster_bwd.hip", "adam.hip", "project.hip", "loss.hip",
           "tile_depth.hip"]
ARCH = os.environ.get("GSR_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compiles every source into libgsr.so (always recompiles). Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and not any(t in ln for t in noise)]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
