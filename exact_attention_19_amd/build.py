"""Build the HIP library ``libattn.so`` in-tree for gfx950.

The library is built with hipcc straight from ``csrc/*.hip``; it exports the
C ABI declared in ``include/attn.h``.  All HIP code is compiled with packed
fp32 arithmetic disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip")]
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libattn.so")


def build_command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, *SOURCES, "-o", out]


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into libattn.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libattn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
