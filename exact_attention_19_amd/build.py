"""Build the HIP library ``libattn.so`` in-tree for gfx950.

The library is built with hipcc straight from ``csrc/*.hip``; it exports the
C ABI declared in ``include/attn.h``.  All HIP code is compiled with packed
fp32 arithmetic disabled (``-packed-fp32-ops``).

    python -m exact_attention_19_amd.build                # libattn.so in the package
    python -m exact_attention_19_amd.build --sanitize     # host ASan/UBSan, _build/sanitize/
    python -m exact_attention_19_amd.build --poison-lds   # LDS poisoned with NaN, libattn_poison.so
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


# Host-side sanitizer build (CPU checks only): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host half of every source (argument
# validation, launch plans, workspace sizes); the gfx950 device code is built
# as usual.  The result goes to SANITIZE_LIB, never over LIB.
SANITIZE_DIR = os.path.join(ROOT, "_build", "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libattn.so")
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined",
                       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


# LDS-poison debug build (GPU checks): every kernel fills its LDS with NaN
# bytes before use, so a read of LDS before the kernel wrote it shows up as
# NaN in parity.  The result goes to POISON_LIB (beside LIB, so that it
# travels with the package), never over LIB.
POISON_LIB = os.path.join(os.path.dirname(LIB), "libattn_poison.so")


def build_command(out: str, src: str | None = None, sanitize: bool = False,
                  poison: bool = False) -> list[str]:
    """hipcc for one source (-c, to an object) or, src None, all of them into a
    shared library."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]
    if sanitize:
        cmd += HOST_SANITIZE_FLAGS
    if poison:
        cmd += ["-DATTN_POISON_LDS"]
    if src is not None:
        return cmd + ["-c", src, "-o", out]
    return cmd + ["-shared", *SOURCES, "-o", out]


def build_library(verbose: bool = False, sanitize: bool = False, poison: bool = False) -> str:
    """Compile every HIP source into libattn.so (always recompiles).  The
    sources are compiled in parallel, then linked."""
    if sanitize and poison:
        raise ValueError("the sanitizer and LDS-poison builds are separate")
    lib = SANITIZE_LIB if sanitize else POISON_LIB if poison else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    objs = [tmp + "." + os.path.basename(s) + ".o" for s in SOURCES]
    procs = []
    for s, o in zip(SOURCES, objs):
        cmd = build_command(o, s, sanitize, poison)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                      text=True))
    failed = False
    for p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
    try:
        if failed:
            raise RuntimeError("hipcc failed to compile libattn.so")
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if sanitize:
            link[1:1] = HOST_SANITIZE_FLAGS
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed to link libattn.so")
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build_library(verbose=True, sanitize="--sanitize" in sys.argv,
                        poison="--poison-lds" in sys.argv))
