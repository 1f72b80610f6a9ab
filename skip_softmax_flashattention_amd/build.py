"""Build the HIP library libssa.so for gfx950 in-tree (no JIT cache).

    python -m skip_softmax_flashattention_amd.build

compiles csrc/ssa_fwd.hip (kernels and their C ABI) and csrc/ssa_config.cpp
(host-only configuration helpers) into _lib/libssa.so with hipcc.  The library is
rebuilt every time this runs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ssa_fwd.hip")
SRC_HOST = os.path.join(PKG, "csrc", "ssa_config.cpp")   # host-only configuration helpers
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
OUT = os.path.join(OUT_DIR, "libssa.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command() -> list:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-I" + INCLUDE,
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-o", OUT + ".tmp", SRC, SRC_HOST,
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = command()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libssa.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
