"""GPU parity of the layout and head-size breadth, through the C ABI, against
the fp64 oracle: strided inputs (the (B, H, S, d) layout, q/k/v sliced from a
packed projection, an output written into a wider buffer), and head sizes
32, 96 and 256 next to 64 and 128.  The oracle always sees the logical
(B, S, H, d) tensors, made dense on the CPU.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_19_amd.workloads import Workload, make_inputs
from parity_common import _check_full, _say, half_ulp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _w(name, B, Hq, Hkv, Sq, Sk, d, dt, causal):
    return Workload(name, B, Hq, Hkv, Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("kv_split", [1, 0, 3])
@pytest.mark.parametrize("Sq,Sk,causal,dt,Hq,Hkv", [
    (300, 300, True, "bf16", 8, 2), (129, 700, True, "f16", 4, 4),
    (700, 129, True, "bf16", 8, 1), (257, 333, False, "f16", 6, 3)])
def test_bhsd_layout(Sq, Sk, causal, dt, Hq, Hkv, kv_split):
    from exact_attention_19_amd import attn_fwd_strided
    w = _w(f"bhsd_{Sq}_{Sk}", 2, Hq, Hkv, Sq, Sk, 128, dt, causal)
    q, k, v = make_inputs(w, seed=Sq + Sk)
    # (B, H, S, d) copies on the device
    qh, kh, vh = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
    _say(f"[gpu] attn_fwd_strided bhsd {w.name} {dt} causal={causal} kv_split={kv_split}")
    o, lse = attn_fwd_strided(qh, kh, vh, scale=w.scale, causal=causal, layout="bhsd",
                              kv_split=kv_split)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (2, Hq, Sq, 128)
    _check_full(w, q, k, v, o.transpose(1, 2).cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_qkv_projection(causal):
    """q, k, v as head slices of one (B, S, Hq + 2 Hkv, d) tensor (Sq = Sk)."""
    from exact_attention_19_amd import attn_fwd_strided
    B, S, Hq, Hkv, d = 2, 333, 8, 2, 128
    w = _w("packed", B, Hq, Hkv, S, S, d, "bf16", causal)
    q, k, v = make_inputs(w, seed=7)
    packed = torch.cat([q, k, v], dim=2).cuda()  # (B, S, Hq + 2 Hkv, d)
    qs, ks, vs = packed[:, :, :Hq], packed[:, :, Hq:Hq + Hkv], packed[:, :, Hq + Hkv:]
    assert not qs.is_contiguous()
    _say(f"[gpu] attn_fwd_strided packed causal={causal}")
    o, lse = attn_fwd_strided(qs, ks, vs, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_k_and_v_with_different_strides_and_strided_output():
    """k in (B, S, H, d), v in (B, H, S, d) (as logical views), and o written
    into the first half of a wider buffer whose second half must stay."""
    from exact_attention_19_amd import attn_fwd_strided
    B, Sq, Sk, Hq, Hkv, d = 2, 200, 450, 8, 4, 64
    w = _w("mixed", B, Hq, Hkv, Sq, Sk, d, "f16", True)
    q, k, v = make_inputs(w, seed=8)
    vg = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)  # logical (B, Sk, Hkv, d)
    wide = torch.full((B, Sq, Hq, 2 * d), 5.0, dtype=torch.float16, device="cuda")
    out = wide[..., :d]
    for kv_split in (1, 4):
        _say(f"[gpu] attn_fwd_strided mixed strides kv_split={kv_split}")
        o, lse = attn_fwd_strided(q.cuda(), k.cuda(), vg, scale=w.scale, causal=True, out=out,
                                  kv_split=kv_split)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr()
        assert torch.all(wide[..., d:] == 5.0)
        _check_full(w, q, k, v, out.cpu(), lse.cpu(), strict=False)


def test_strided_dense_equals_attn_fwd_bit_for_bit():
    from exact_attention_19_amd import attn_fwd, attn_fwd_strided
    w = _w("dense_eq", 1, 16, 4, 513, 1000, 128, "bf16", True)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=9))
    o1, l1 = attn_fwd(q, k, v, scale=w.scale, causal=True)
    o2, l2 = attn_fwd_strided(q, k, v, scale=w.scale, causal=True, kv_split=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _head_size_cases():
    cases = []
    for d in (32, 96, 256):
        for dt in ("f16", "bf16"):
            cases.append((d, dt, 1, 128, 128, False, 2, 2))
            cases.append((d, dt, 2, 333, 517, True, 8, 2))
            cases.append((d, dt, 1, 517, 300, True, 4, 4))
            cases.append((d, dt, 1, 1, 700, True, 8, 1))
    return cases


@pytest.mark.parametrize("d,dt,B,Sq,Sk,causal,Hq,Hkv", _head_size_cases())
def test_head_sizes(d, dt, B, Sq, Sk, causal, Hq, Hkv):
    from exact_attention_19_amd import attn_fwd
    w = _w(f"hd{d}_{dt}_{Sq}_{Sk}", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=d + Sq)
    _say(f"[gpu] attn_fwd head size {d} {w.name} causal={causal}")
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_head_sizes_with_key_split(d):
    from exact_attention_19_amd import attn_fwd_split
    w = _w(f"hd{d}_split", 1, 8, 2, 300, 2000, d, "bf16", True)
    q, k, v = make_inputs(w, seed=d)
    _say(f"[gpu] attn_fwd_split head size {d}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True,
                            kv_split=5)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_merge_head_sizes():
    """attn_merge at d = 96 (a row of 24 threads) against numpy in fp64."""
    from exact_attention_19_amd import attn_merge
    from oracle import merge_partials_oracle
    r = np.random.default_rng(12)
    P, B, Sq, Hq, d = 3, 2, 37, 3, 96
    op = r.standard_normal((P, B, Sq, Hq, d)).astype(np.float32)
    lp = (2 * r.standard_normal((P, B, Hq, Sq))).astype(np.float32)
    o_ref, lse_ref = merge_partials_oracle(op.astype(np.float64), lp.astype(np.float64))
    o, lse = attn_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(),
                        dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.abs(o.double().cpu().numpy() - o_ref).max() <= 2e-3
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= 1e-4


@pytest.mark.parametrize("kv_split", [1, 3])
@pytest.mark.parametrize("Sq,Sk,causal,dt", [(200, 333, True, "bf16"), (129, 64, False, "f16"),
                                             (77, 1000, True, "f16")])
def test_kv_broadcast_along_seq(Sq, Sk, causal, dt, kv_split):
    """k and v expanded along the key axis (row stride 0): every key is the
    same row, read whole through the tile descriptors."""
    from exact_attention_19_amd import attn_fwd_strided
    w = _w(f"kv_bcast_{Sq}_{Sk}", 2, 8, 2, Sq, Sk, 128, dt, causal)
    q, k, v = make_inputs(w, seed=Sq + 3 * Sk)
    k1, v1 = k[:, :1], v[:, :1]
    kx, vx = k1.cuda().expand(-1, Sk, -1, -1), v1.cuda().expand(-1, Sk, -1, -1)
    assert kx.stride(1) == 0
    _say(f"[gpu] attn_fwd_strided K/V broadcast along S {w.name} kv_split={kv_split}")
    o, lse = attn_fwd_strided(q.cuda(), kx, vx, scale=w.scale, causal=causal, kv_split=kv_split)
    torch.cuda.synchronize()
    kd, vd = k1.expand(-1, Sk, -1, -1).contiguous(), v1.expand(-1, Sk, -1, -1).contiguous()
    _check_full(w, q, kd, vd, o.cpu(), lse.cpu(), strict=False)


def test_kv_overlapping_rows():
    """k and v views whose rows overlap (row stride 64 elements < d = 128):
    key j is elements [64 j, 64 j + 128) of one flat buffer."""
    from exact_attention_19_amd import attn_fwd_strided
    B, Sq, Sk, Hq, Hkv, d = 1, 150, 300, 4, 1, 128
    w = _w("kv_overlap", B, Hq, Hkv, Sq, Sk, d, "bf16", True)
    q, _, _ = make_inputs(w, seed=21)
    g = torch.Generator().manual_seed(22)
    flat_k = torch.randn(64 * (Sk + 1), generator=g).to(torch.bfloat16)
    flat_v = torch.randn(64 * (Sk + 1), generator=g).to(torch.bfloat16)
    fk, fv = flat_k.cuda(), flat_v.cuda()
    kx = fk.as_strided((B, Sk, Hkv, d), (0, 64, 0, 1))
    vx = fv.as_strided((B, Sk, Hkv, d), (0, 64, 0, 1))
    _say("[gpu] attn_fwd_strided overlapping K/V rows")
    o, lse = attn_fwd_strided(q.cuda(), kx, vx, scale=w.scale, causal=True, kv_split=1)
    torch.cuda.synchronize()
    kd = flat_k.as_strided((B, Sk, Hkv, d), (0, 64, 0, 1)).contiguous()
    vd = flat_v.as_strided((B, Sk, Hkv, d), (0, 64, 0, 1)).contiguous()
    _check_full(w, q, kd, vd, o.cpu(), lse.cpu(), strict=False)


def test_binding_rejects_bad_buffers_before_any_launch():
    """Caller-given outputs and workspaces of the wrong shape, dtype, layout
    or device raise before the library is called."""
    from exact_attention_19_amd import (attn_bwd, attn_decode_paged, attn_fwd, attn_fwd_split,
                                        attn_fwd_strided, attn_merge)
    w = _w("bad_bufs", 1, 4, 2, 64, 64, 64, "bf16", True)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=1))
    lse_ok = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")
    bad_outs = [torch.empty(1, 64, 4, 32, dtype=torch.bfloat16, device="cuda"),   # shape
                torch.empty_like(q, dtype=torch.float16),                           # dtype
                torch.empty(1, 64, 4, 128, dtype=torch.bfloat16, device="cuda")[..., :64],
                torch.empty(q.shape, dtype=torch.bfloat16)]                         # host
    for out in bad_outs:
        for fn in (attn_fwd, attn_fwd_split):
            with pytest.raises(ValueError):
                fn(q, k, v, causal=True, out=out)
    for lse in (torch.empty((1, 4, 64), dtype=torch.float32),                       # host
                torch.empty((1, 4, 63), dtype=torch.float32, device="cuda")):
        with pytest.raises(ValueError):
            attn_fwd(q, k, v, causal=True, lse=lse)
        with pytest.raises(ValueError):
            attn_fwd_strided(q, k, v, causal=True, lse=lse)
    with pytest.raises(ValueError):
        attn_fwd_split(q, k, v, causal=True, kv_split=2,
                       workspace=torch.empty(1 << 20, dtype=torch.uint8))
    o, lse = attn_fwd(q, k, v, causal=True)
    do = torch.randn_like(q)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError):
            attn_bwd(q, k, v, o, lse, do, causal=True, **{name: torch.empty(k.shape if name != "dq"
                                                                            else q.shape,
                                                                            dtype=q.dtype)})
    with pytest.raises(ValueError):
        attn_bwd(q, k, v, o, lse.cpu(), do, causal=True)
    with pytest.raises(ValueError):
        attn_bwd(q, k, v, o, lse, do, causal=True, workspace=torch.empty(4096, dtype=torch.uint8))
    parts = torch.zeros((2, 1, 64, 4, 64), dtype=torch.float32, device="cuda")
    plse = torch.zeros((2, 1, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        attn_merge(parts, plse, out=torch.empty((1, 64, 4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        attn_merge(parts, plse, lse=torch.empty((1, 4, 64), dtype=torch.float32))
    qd = q[:, :1].contiguous()
    pool = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    lens = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        attn_decode_paged(qd, pool, pool, table, lens, out=torch.empty(qd.shape, dtype=qd.dtype))
    torch.cuda.synchronize()


# ------------------------------------------------------------ padded head sizes
#
# Head sizes that are multiples of 8 but not of 32 (and 160, 192, 200) run on
# the kernel of the next built size (32, 64, 96, 128, 192, 256): the columns
# past d load as zeros and are not stored.

PADDED = (8, 40, 80, 104, 160, 192, 200)


def _padded_cases():
    cases = []
    for d in PADDED:
        for dt in ("f16", "bf16"):
            cases.append((d, dt, 2, 333, 517, True, 8, 2))     # causal, offset, GQA 4
            cases.append((d, dt, 1, 200, 130, True, 4, 4))     # rows with no key
        cases.append((d, "bf16", 1, 129, 300, False, 6, 3))
        cases.append((d, "f16", 1, 1, 700, True, 8, 1))        # decode kernel
    return cases


@pytest.mark.parametrize("d,dt,B,Sq,Sk,causal,Hq,Hkv", _padded_cases())
def test_padded_head_sizes(d, dt, B, Sq, Sk, causal, Hq, Hkv):
    from exact_attention_19_amd import attn_fwd
    w = _w(f"pad{d}_{dt}_{Sq}_{Sk}", B, Hq, Hkv, Sq, Sk, d, dt, causal)
    q, k, v = make_inputs(w, seed=3 * d + Sq)
    _say(f"[gpu] attn_fwd padded head size {d} {w.name} causal={causal}")
    # outputs start as NaN: every element of o must be written, none past d
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal, out=o)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("d", [40, 80, 136, 160, 168, 200, 248])
def test_padded_head_sizes_split_and_strided(d):
    """The key split (partial states of the padded size, merged into d
    columns) and strided views whose rows are d long inside wider rows: the
    columns past d of the wider rows are NaN and must never be read."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_strided
    w = _w(f"pad{d}_split", 1, 8, 2, 300, 2000, d, "bf16", True)
    q, k, v = make_inputs(w, seed=d + 1)
    _say(f"[gpu] attn_fwd_split padded head size {d}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True, kv_split=5)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)
    wide = 256 + 64
    def embed(t):
        x = torch.full(t.shape[:3] + (wide,), float("nan"), dtype=t.dtype)
        x[..., :d] = t
        return x.cuda()[..., :d]
    qs, ks, vs = embed(q), embed(k), embed(v)
    assert qs.stride(2) == wide
    _say(f"[gpu] attn_fwd_strided padded head size {d} in rows of {wide}")
    o2, lse2 = attn_fwd_strided(qs, ks, vs, scale=w.scale, causal=True, kv_split=0)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o2.cpu(), lse2.cpu(), strict=False)


@pytest.mark.parametrize("d", [40, 200, 256])
def test_padded_and_large_head_sizes_paged_decode(d):
    from exact_attention_19_amd import attn_decode_paged
    from exact_attention_19_amd.workloads import make_paged_cache
    from oracle import attn_decode_paged_oracle
    w = _w(f"paged_d{d}", 3, 16, 4, 2, 1000, d, "bf16", True)
    q, k, v = make_inputs(w, seed=d)
    lens = [1000, 517, 33]
    kp, vp, table, seqlens = make_paged_cache(k, v, lens, 64, seed=1)
    _say(f"[gpu] attn_decode_paged head size {d}")
    o, lse = attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), seqlens.cuda(),
                               scale=w.scale, causal=True, max_seqlen=1000)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_decode_paged_oracle(q, kp, vp, table, seqlens, w.scale, True, 1000)
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False, ref=(o_ref, lse_ref))


def test_merge_padded_head_size():
    """attn_merge at d = 40 (parts with rows of 40 floats) against numpy fp64."""
    from exact_attention_19_amd import attn_merge
    from oracle import merge_partials_oracle
    r = np.random.default_rng(13)
    P, B, Sq, Hq, d = 4, 2, 29, 3, 40
    op = r.standard_normal((P, B, Sq, Hq, d)).astype(np.float32)
    lp = (2 * r.standard_normal((P, B, Hq, Sq))).astype(np.float32)
    o_ref, lse_ref = merge_partials_oracle(op.astype(np.float64), lp.astype(np.float64))
    o, lse = attn_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(),
                        dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the merge is fp32: the error is the rounding of O to bf16 (half an ulp)
    # plus fp32 arithmetic
    diff = np.abs(o.double().cpu().numpy() - o_ref)
    assert np.all(diff <= half_ulp(o_ref, "bf16") + 1e-5 * (1 + np.abs(o_ref)))
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= 1e-4


@pytest.mark.parametrize("d", [8, 40, 136, 200])
def test_padded_head_sizes_decode_strided(d):
    """The decode kernel (one query row per head) on rows of d inside wider
    NaN-filled rows: no column past d may be read."""
    from exact_attention_19_amd import attn_fwd_plan, attn_fwd_strided
    from exact_attention_19_amd.binding import ATTN_DTYPE_BF16
    w = _w(f"pad{d}_decode_strided", 2, 16, 4, 1, 900, d, "bf16", True)
    assert attn_fwd_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, d, 1, ATTN_DTYPE_BF16)["decode"] == 1
    q, k, v = make_inputs(w, seed=d + 5)
    wide = 264
    def embed(t):
        x = torch.full(t.shape[:3] + (wide,), float("nan"), dtype=t.dtype)
        x[..., :d] = t
        return x.cuda()[..., :d]
    for kv_split in (1, 0):
        _say(f"[gpu] attn_fwd_strided decode kernel, head size {d} in rows of {wide}, "
             f"kv_split={kv_split}")
        o, lse = attn_fwd_strided(embed(q), embed(k), embed(v), scale=w.scale, causal=True,
                                  kv_split=kv_split)
        torch.cuda.synchronize()
        _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("d,Sq,Sk,causal,kv_split", [
    (256, 700, 700, True, 1),
    (256, 300, 2000, True, 3),
    (248, 513, 1000, False, 1),
    (200, 333, 1500, True, 0),
    (192, 1280, 1536, True, 2),
    (176, 300, 2000, True, 3),
    (184, 513, 1000, False, 0),
    (192, 64, 4096, False, 0),
])
def test_f16_head_size_256_key_halves(d, Sq, Sk, causal, kv_split):
    """fp16 at padded head sizes 192 and 256 runs the key halves (unsplit and
    in the pieces of a key split)."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    from exact_attention_19_amd.binding import ATTN_DTYPE_F16
    w = _w(f"f16_hd{d}_kh_{Sq}_{Sk}", 2, 8, 2, Sq, Sk, d, "f16", causal)
    plan = attn_fwd_split_plan(w.B, Sq, Sk, w.Hq, w.Hkv, d, int(causal), ATTN_DTYPE_F16, kv_split)
    assert plan["key_halves"] == 1
    q, k, v = make_inputs(w, seed=d + Sq + Sk)
    _say(f"[gpu] attn_fwd_split fp16 head size {d} {w.name} kv_split={kv_split} "
         f"(pieces {plan['pieces']})")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal,
                            kv_split=kv_split)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)
