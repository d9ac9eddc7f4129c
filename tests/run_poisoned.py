"""GPU parity suites against the LDS-poison debug build of libattn.so.

The debug build (``python -m exact_attention_19_amd.build --poison-lds``, made
beforehand on the build machine: ``libattn_poison.so`` beside ``libattn.so``)
starts every kernel (forward, two-group forward, key split, decode, backward)
by filling each of its LDS arrays with 0xFF bytes, a NaN in fp32, fp16 and
bf16, before its first tile load.  A kernel that reads LDS it has not written
first then produces NaN, which the parity tests' finiteness and oracle checks
catch.  This runs the GPU test modules (``tests/test_*_gpu.py`` unless test
files are given) with the binding pointed at that build (ATTN_LIBRARY).  Needs
an MI355X.

    python tests/run_poisoned.py [test files] [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main() -> int:
    from exact_attention_19_amd.build import POISON_LIB as lib
    if not os.path.exists(lib):
        print(f"{lib} is missing: build it first with "
              "python -m exact_attention_19_amd.build --poison-lds", file=sys.stderr)
        return 2
    args = sys.argv[1:]
    if not any(a.endswith(".py") for a in args):
        files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_*_gpu.py")))
        args = files + args
    env = dict(os.environ, ATTN_LIBRARY=lib)
    cmd = [sys.executable, "-u", "-m", "pytest", "-q", "-x", "-m", "gpu", "-p", "no:cacheprovider",
           "--timeout", "600", "--timeout-method", "thread", *args]
    print("LDS-poison run:", " ".join(cmd), f"\n  ATTN_LIBRARY={lib}", flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())
