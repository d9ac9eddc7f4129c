"""Checks shared by the GPU parity tests (not a test module itself).

Tolerances (max |delta O| against the exact fp64 result): 2e-3 for fp16 and
1e-2 for bf16 inputs; LSE within 1e-3.
"""
import sys

import numpy as np

from oracle import attn_fwd_oracle

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3

# Per-case records that the session summary prints (tests/conftest.py):
#   FLAT_EXCESS: cases checked with the output-rounding bound, with how many
#     elements exceed the flat tolerance, the worst excess and the output-
#     rounding floor (half an ulp of the exact value) at that element;
#   FULL_SIZE: max |dO| and |dLSE| over every row of a full-size workload.
FLAT_EXCESS = []
FULL_SIZE = []


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def half_ulp(x, dtype):
    """Half the spacing of the output format at |x| (the output-rounding floor:
    11 significant bits for fp16, 8 for bf16; subnormal fp16 spacing 2^-24)."""
    p = 11 if dtype == "f16" else 8
    a = np.maximum(np.abs(x), 2.0 ** -14 if dtype == "f16" else 2.0 ** -126)
    e = np.floor(np.log2(a))
    return 0.5 * 2.0 ** (e - (p - 1))


def allowed_error(o_ref, dtype, strict):
    """The workloads of the headline table use the flat tolerance (2e-3 fp16,
    1e-2 bf16).  The extra edge cases use a bound derived from the arithmetic:
    the flat tolerance, except where the exact output is so large that its own
    rounding to the output format (half an ulp) exceeds half of it; there the
    bound is that half-ulp plus half the flat tolerance for the arithmetic."""
    tol = TOL_O[dtype]
    if strict:
        return np.full(o_ref.shape, tol)
    hu = half_ulp(o_ref, dtype)
    return np.where(hu <= tol / 2, tol, hu + tol / 2)


def record_flat_excess(name, dtype, diff, o_ref):
    """Count the elements whose error exceeds the flat tolerance (allowed by
    the output-rounding bound) and keep the worst with its floor."""
    tol = TOL_O[dtype]
    over = diff > tol
    n = int(over.sum())
    if n:
        at = np.unravel_index(np.argmax(np.where(over, diff, -1.0)), diff.shape)
        floor = float(half_ulp(o_ref[at], dtype))
        FLAT_EXCESS.append((name, n, int(diff.size), float(diff[at]), float(o_ref[at]), floor))
        _say(f"{name}: {n} of {diff.size} elements over the flat {tol:g}; worst "
             f"|dO| = {diff[at]:.4e} at |O| = {abs(o_ref[at]):.3f} (output-rounding floor "
             f"{floor:.4e})")
    else:
        FLAT_EXCESS.append((name, 0, int(diff.size), float(diff.max()), 0.0, 0.0))


def _check_full(w, q, k, v, o, lse, strict=True, ref=None):
    """ref: the oracle's (o, lse) for these inputs, if already computed."""
    o_ref, lse_ref = ref if ref is not None else attn_fwd_oracle(q, k, v, w.scale, w.causal)
    diff = np.abs(o.double().numpy() - o_ref)
    err = diff.max()
    assert np.isfinite(o.float().numpy()).all()
    bound = allowed_error(o_ref, w.dtype, strict)
    worst = np.unravel_index(np.argmax(diff - bound), diff.shape)
    if not strict:
        record_flat_excess(w.name, w.dtype, diff, o_ref)
    assert np.all(diff <= bound), (
        f"{w.name}: max|dO| = {err}; worst excess at {worst}: "
        f"|dO| = {diff[worst]}, bound {bound[worst]}, ref {o_ref[worst]}")
    if lse is not None:
        lg = lse.double().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin), "empty rows must give -inf"
        assert np.all(np.isneginf(lg[~fin]))
        if fin.any():
            el = np.abs(lg[fin] - lse_ref[fin]).max()
            assert el <= TOL_LSE, f"{w.name}: max|dLSE| = {el}"
        # empty rows give O = 0
        empty = ~fin  # (B, Hq, Sq)
        ob = o.float().numpy()
        for b, h, i in zip(*np.nonzero(empty)):
            assert np.all(ob[b, i, h] == 0)
    return err
