"""GPU parity of the forward's workgroup shapes for launches of at most one
4-wave workgroup per CU, against the fp64 oracle.

Key halves (attn_fwd, and attn_fwd_split when it does not split): the 4
waves of a workgroup are 2 row waves x 2 key halves.  Both waves of a row
wave take the same 32 query rows, one the first and one the second 32 keys
of every 64-key tile, each with its own online-softmax state; at the end the
two states are combined through LDS with the online-softmax rescale
("FlashAttention personal implementation notes", section "Online Softmax":
the max, the rescale factor on the denominator and the output), each wave
finishing half of the output columns (at d = 32, one column block, one wave
finishes them all).

Two groups (the pieces of a key split): a workgroup is two 4-wave groups over
alternate key tiles of the same query rows, merged the same way; a group
whose share is one tile short runs a filler tile whose keys are all masked.

Every case asserts the plan it means to test, then compares every element
with the oracle (the output-rounding bound of the edge cases: the flat 2e-3
fp16 / 1e-2 bf16, widened to half an ulp + half the flat tolerance where the
exact value is so large that its own rounding exceeds half of it; LSE
within 1e-3).
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


# (B, Hq, Hkv, Sq, Sk, d, dtype, causal): at most 256 row blocks of 128 rows
# (or of 32 rows of up to 4 GQA heads), >= 8 tiles in the longest
CASES = [
    (1, 8, 8, 1100, 1100, 128, "f16", True),     # ragged query tail, 18 tiles
    (2, 4, 2, 200, 520, 128, "bf16", False),     # 9 tiles; GQA 2
    (1, 8, 2, 300, 1000, 128, "bf16", True),     # causal offset 700, 13..16 tiles
    (1, 4, 4, 1000, 1000, 40, "f16", True),      # padded head size 40 -> 64
    (1, 4, 1, 700, 900, 120, "bf16", True),      # padded 120 -> 128, GQA 4
    (1, 6, 3, 513, 1031, 64, "f16", False),      # 17 tiles, ragged keys
    (1, 8, 8, 1000, 600, 96, "bf16", True),      # Sq > Sk: rows with no key; 3 column blocks
    (4, 16, 16, 256, 512, 32, "f16", True),      # d = 32 (one column block), 8 tiles exactly
    (1, 16, 16, 40, 2048, 128, "f16", True),     # 40 rows: row wave 1 mostly past Sq
    (2, 32, 4, 300, 900, 64, "bf16", True),      # GQA 8: two heads per workgroup, snake per XCD
    (3, 6, 2, 333, 700, 128, "f16", False),      # GQA 3, columns not a multiple of 8: no XCD order
]


def _workload(tag, B, Hq, Hkv, Sq, Sk, d, dt, causal):
    return Workload(f"{tag}_b{B}_h{Hq}_{Hkv}_sq{Sq}_sk{Sk}_d{d}_{dt}_c{int(causal)}", B, Hq, Hkv,
                    Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,causal", CASES)
def test_key_halves_parity(B, Hq, Hkv, Sq, Sk, d, dt, causal):
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    plan = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt))
    assert plan["key_halves"] == 1 and plan["threads"] == 256, plan
    w = _workload("kh", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=Sq + 3 * Sk + d)
    _say(f"[gpu] attn_fwd (key halves) {w.name} {plan}")
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,causal", [CASES[i] for i in (0, 2, 3, 4, 5)])
def test_two_groups_parity(B, Hq, Hkv, Sq, Sk, d, dt, causal):
    """The same shapes cut into two key pieces of at least 8 tiles: each
    piece runs two groups (one of them a filler tile short where the piece
    has an odd number of tiles)."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    plan = attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt), 2)
    assert plan["threads"] == 512 and plan["pieces"] == 2, plan
    w = _workload("ng2", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=Sq + 3 * Sk + d)
    _say(f"[gpu] attn_fwd_split (two groups) {w.name} {plan}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal,
                            kv_split=2)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("kv_split", [2, 3])
def test_two_groups_with_key_split(kv_split):
    """Pieces of a key split run two groups when they are long enough; the
    last piece of a block can hold an odd number of tiles (filler)."""
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


def test_automatic_split_over_key_halves():
    """An automatic split into 8 pieces is kept over the key halves (it is
    the faster of the two there); the result matches the oracle."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    B, Hq, Hkv, Sq, Sk, d, dt, causal = 1, 8, 8, 512, 2048, 128, "f16", False
    plan = attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt), 0)
    assert plan["pieces"] == 8 and plan["key_halves"] == 0, plan
    w = _workload("auto8", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=8)
    _say(f"[gpu] attn_fwd_split (automatic) {w.name} {plan}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_short_rows_take_four_row_waves():
    """Below 8 tiles in the longest block the plan keeps 4 row waves of one
    group; the result matches the oracle."""
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    B, Hq, Hkv, Sq, Sk, d, dt, causal = 2, 16, 16, 256, 256, 128, "f16", True
    plan = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, 1, _code(dt))
    assert plan["threads"] == 256 and plan["key_halves"] == 0, plan
    w = Workload("rows4_short", B, Hq, Hkv, Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=5)
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("d,split", [(128, 1), (72, 1), (96, 1), (32, 1), (128, 2)])
def test_no_writes_outside_outputs(d, split):
    """Canaries around O and LSE stay untouched, and every O element and LSE
    entry between them is written: key halves at d = 128, 72 (on the
    96-column kernel, O dense with 72 columns, so a column past d written by
    mistake would land on the next row or on a canary), 96 (three column
    blocks split 1 + 2 between the key halves) and 32 (one wave finishes the
    rows); two groups on the pieces of a split at d = 128 (1100 keys)."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    Sk = 700 if split == 1 else 1100  # pieces of 10 tiles: two groups
    w = Workload(f"canary_d{d}_s{split}", 1, 8, 2, 333, Sk, d, "bf16", True, 1.0 / math.sqrt(d))
    plan = attn_fwd_split_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, d, 1, _code("bf16"), split)
    if split == 1:
        assert plan["key_halves"] == 1, plan
    else:
        assert plan["threads"] == 512 and plan["pieces"] == 2, plan
    q, k, v = (t.cuda() for t in make_inputs(w, seed=11))
    n_o = w.B * w.Sq * w.Hq * w.d
    pad = 4096
    obuf = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    n_l = w.B * w.Hq * w.Sq
    lbuf = torch.full((n_l + 2 * pad,), 777.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n_o].view(w.B, w.Sq, w.Hq, w.d)
    lse = lbuf[pad:pad + n_l].view(w.B, w.Hq, w.Sq)
    attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=split, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n_o:] == 1234.0)
    assert torch.all(lbuf[:pad] == 777.0) and torch.all(lbuf[pad + n_l:] == 777.0)
    assert torch.all(lse != 777.0) and torch.all(o != 1234.0)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,causal", [
    (1, 8, 2, 700, 900, 192, "bf16", True),      # GQA 4: one head per row wave
    (2, 4, 4, 333, 517, 192, "f16", True),       # MHA, ragged rows and keys
    (1, 16, 2, 300, 1000, 160, "bf16", True),    # GQA 8, padded 160 -> 192
    (1, 6, 3, 129, 300, 176, "f16", False),      # GQA 2, padded 176 -> 192
    (1, 4, 4, 200, 130, 192, "bf16", True),      # Sq > Sk: rows with no key
])
def test_eight_wave_key_halves_d192(B, Hq, Hkv, Sq, Sk, d, dt, causal):
    """At padded head size 192 an unsplit call runs 8-wave workgroups: 4 row
    waves x 2 key halves over one set of tile buffers (two waves per SIMD),
    the 8 waves loading alternate column blocks of each tile and merging the
    key halves through two slots per tile buffer."""
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    plan = attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), _code(dt))
    assert plan["key_halves"] == 1 and plan["threads"] == 512, plan
    w = _workload("kh8", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=Sq + Sk + d)
    _say(f"[gpu] attn_fwd (8-wave key halves) {w.name} {plan}")
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal, out=o)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_eight_wave_key_halves_no_writes_outside_outputs():
    """Canaries around O and LSE at d = 184 on the 8-wave d = 192 kernel: O
    is dense with 184 columns, so a column past d written by mistake would
    land on the next row or on a canary."""
    from exact_attention_19_amd import attn_fwd
    from exact_attention_19_amd.binding import attn_fwd_plan
    d = 184
    w = Workload("kh8_canary", 1, 8, 2, 333, 700, d, "bf16", True, 1.0 / math.sqrt(d))
    assert attn_fwd_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, d, 1, _code("bf16"))["threads"] == 512
    q, k, v = (t.cuda() for t in make_inputs(w, seed=12))
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


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_eight_wave_key_halves_strided(layout):
    """Strided views at d = 192, unsplit: q, k, v as (B, H, S, d) transposes
    or as slices of wider rows; the 8-wave workgroups read them through the
    element strides."""
    from exact_attention_19_amd import attn_fwd_strided, attn_fwd_split_plan
    B, Hq, Hkv, Sq, Sk, d = 2, 8, 4, 300, 700, 192
    plan = attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, 1, _code("bf16"), 1)
    assert plan["key_halves"] == 1 and plan["threads"] == 512, plan
    w = _workload(f"kh8_strided_{layout}", B, Hq, Hkv, Sq, Sk, d, "bf16", True)
    q, k, v = make_inputs(w, seed=21)
    if layout == "bhsd":
        qs, ks, vs = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
    else:
        wide = 256
        def embed(t):
            x = torch.full(t.shape[:3] + (wide,), float("nan"), dtype=t.dtype)
            x[..., :d] = t
            return x.cuda()[..., :d]
        qs, ks, vs = embed(q), embed(k), embed(v)
    _say(f"[gpu] attn_fwd_strided (8-wave key halves) {w.name} {plan}")
    o, lse = attn_fwd_strided(qs, ks, vs, scale=w.scale, causal=True, layout=layout, kv_split=1)
    torch.cuda.synchronize()
    if layout == "bhsd":
        o = o.transpose(1, 2)
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)
