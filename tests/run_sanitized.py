"""CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-side sanitizer build of libattn.so (the argument validation,
launch plans and workspace sizes of every entry point; the gfx950 device code
is built as usual) and the sanitizer build of the fp64 oracle, both into
_build/sanitize/, then runs ``pytest -m "not gpu"`` with those builds loaded in
place of the normal ones and the clang sanitizer runtime preloaded into the
Python process.  Any heap overflow, use after free or undefined behaviour in
either library aborts the run.  CPU only: nothing here touches a GPU.

    python tests/run_sanitized.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def runtime() -> str:
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang's AddressSanitizer runtime is not installed")
    return libs[-1]


def main() -> int:
    from exact_attention_19_amd.build import build_library
    from oracle import build_oracle
    lib = build_library(sanitize=True)
    olib = build_oracle(force=True, sanitize=True)
    env = dict(os.environ)
    env.update({
        "ATTN_LIBRARY": lib,
        "ATTN_ORACLE_LIBRARY": olib,
        "LD_PRELOAD": runtime(),
        # Python and torch keep memory until exit: leak reports would be noise
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    print("sanitized run:", " ".join(cmd), flush=True)
    print(f"  ATTN_LIBRARY={lib}\n  ATTN_ORACLE_LIBRARY={olib}\n  LD_PRELOAD={env['LD_PRELOAD']}",
          flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
