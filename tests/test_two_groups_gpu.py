"""GPU parity of the two-group forward workgroups against the fp64 oracle.

When a launch has at most one workgroup per CU and its longest row block
holds at least 8 key tiles, each workgroup runs two 4-wave groups over
alternate key tiles of the same query rows and merges their online-softmax
states through LDS at the end ("FlashAttention personal implementation
notes", section "Online Softmax": the max, the rescale factor on the
denominator and the output).  A group whose share is one tile short runs a
filler tile whose keys are all masked.  Every case here asserts that its
plan takes the two-group workgroups, then compares every element with the
oracle (the output-rounding bound of the edge cases: the flat 2e-3 fp16 /
1e-2 bf16, widened to half an ulp + half the flat tolerance where the exact
value is so large that its own rounding exceeds half of it; LSE within 1e-3).
"""
import math

import pytest
import torch

from exact_attention_19_amd.workloads import Workload, make_inputs
from parity_common import _check_full, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _code(dt):
    from exact_attention_19_amd.binding import ATTN_DTYPE_BF16, ATTN_DTYPE_F16
    return ATTN_DTYPE_BF16 if dt == "bf16" else ATTN_DTYPE_F16


# (B, Hq, Hkv, Sq, Sk, d, dtype, causal): at most 256 row blocks, >= 8 tiles
CASES = [
    (1, 8, 8, 1100, 1100, 128, "f16", True),     # ragged query tail, 18 tiles
    (2, 4, 2, 200, 520, 128, "bf16", False),     # 9 tiles: group 1 runs a filler
    (1, 8, 2, 300, 1000, 128, "bf16", True),     # causal offset 700, 13..16 tiles
    (1, 4, 4, 1000, 1000, 40, "f16", True),      # padded head size 40 -> 64
    (1, 4, 1, 700, 900, 120, "bf16", True),      # padded 120 -> 128, GQA 4
    (1, 6, 3, 513, 1031, 64, "f16", False),      # 17 tiles, ragged keys
    (1, 8, 8, 1000, 600, 96, "bf16", True),      # Sq > Sk: rows with no key
    (4, 16, 16, 256, 512, 32, "f16", True),      # d = 32, 8 tiles exactly
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,causal", CASES)
def test_two_groups_parity(B, Hq, Hkv, Sq, Sk, d, dt, causal):
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    plan = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt))
    assert plan["threads"] == 512, plan
    w = Workload(f"ng2_b{B}_h{Hq}_{Hkv}_sq{Sq}_sk{Sk}_d{d}_{dt}_c{int(causal)}", B, Hq, Hkv,
                 Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=Sq + 3 * Sk + d)
    _say(f"[gpu] attn_fwd (two groups) {w.name} {plan}")
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("kv_split", [2, 3])
def test_two_groups_with_key_split(kv_split):
    """Pieces of a key split run two groups too when they are long enough;
    the last piece of a block can hold an odd number of tiles (filler)."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    B, Hq, Hkv, Sq, Sk, d, dt, causal = 1, 8, 4, 1100, 1500, 128, "f16", True
    plan = attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt), kv_split)
    assert plan["threads"] == 512 and plan["pieces"] == kv_split, plan
    w = Workload(f"ng2_split{kv_split}", B, Hq, Hkv, Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=kv_split)
    _say(f"[gpu] attn_fwd_split (two groups) {w.name} {plan}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal,
                            kv_split=kv_split)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_two_groups_short_rows_take_one_group():
    """Below 8 tiles in the longest block the plan keeps one 4-wave group;
    both kinds give the same attention to rounding (here: the oracle's)."""
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    B, Hq, Hkv, Sq, Sk, d, dt, causal = 2, 16, 16, 256, 256, 128, "f16", True
    assert attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, 1, _code(dt))["threads"] == 256
    w = Workload("ng1_short", B, Hq, Hkv, Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=5)
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("d", [128, 72])
def test_two_groups_no_writes_outside_outputs(d):
    """Canaries around O and LSE stay untouched, and every O element and LSE
    entry between them is written.  At d = 72 (run on the 96-column kernel)
    O is dense with 72 columns, so a column past d written by mistake would
    land on the next row or on a canary."""
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    w = Workload(f"ng2_canary_d{d}", 1, 8, 2, 333, 700, d, "bf16", True, 1.0 / math.sqrt(d))
    assert attn_fwd_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, d, 1, _code("bf16"))["threads"] == 512
    q, k, v = (t.cuda() for t in make_inputs(w, seed=11))
    n_o = w.B * w.Sq * w.Hq * w.d
    pad = 4096
    obuf = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    n_l = w.B * w.Hq * w.Sq
    lbuf = torch.full((n_l + 2 * pad,), 777.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n_o].view(w.B, w.Sq, w.Hq, w.d)
    lse = lbuf[pad:pad + n_l].view(w.B, w.Hq, w.Sq)
    attn_fwd(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n_o:] == 1234.0)
    assert torch.all(lbuf[:pad] == 777.0) and torch.all(lbuf[pad + n_l:] == 777.0)
    assert torch.all(lse != 777.0) and torch.all(o != 1234.0)
