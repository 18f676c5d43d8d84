"""Build libflce.so (the HIP kernels and the C ABI) in-tree for gfx950, and
the matrix-core ceiling probe bench.py runs for context (mfma_ceiling).

    python lm_head_linear_flce_amd/build.py

Cross-compiles on a machine without a GPU.  Both land next to this file, where
the Python binding loads the library from.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libflce.so")
SOURCES = [os.path.join(CSRC, "flce_api.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("flce_tile.h", "flce_kernels.h")] + \
    [os.path.join(ROOT, "include", "flce.h")]
CEILING = os.path.join(HERE, "mfma_ceiling")
CEILING_SOURCE = os.path.join(CSRC, "mfma_ceiling.hip")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(out: str = LIB):
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # code object v5: loadable by the HIP runtime PyTorch ships as well
        "-mcode-object-version=5",
        # packed fp32 VALU forms stay off (see the design notes)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, *SOURCES,
    ]


def ceiling_command(out: str = CEILING):
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-o", out, CEILING_SOURCE,
    ]


def _run(cmd, out, verbose):
    tmp = out + ".tmp"
    cmd = cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libflce.so and the ceiling probe; returns the library's path."""
    _run(ceiling_command, CEILING, verbose)
    return _run(command, LIB, verbose)


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
