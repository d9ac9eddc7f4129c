"""GPU parity of attn_fwd_causal_offset (causal attention with an explicit
mask offset) against the fp64 oracle: each key shard of a longer causal
problem, given causal_offset = Sk_total - Sq - k0, is the oracle's partial
state over that key range of the full problem, and attn_merge of the shards
is the full causal attention (the single-device half of key sharding).
Prefill and decode shapes, with and without the key split; offsets that
leave every key visible or none.  Tolerances as for the forward, plus the
extra rounding of 16-bit shard outputs in the merged result.

attn_bwd_causal_offset, the backward of a shard given the full problem's O
and LSE: its dK, dV are the slices of the oracle's full-problem gradients,
and the sum of the shards' dQ parts is the full dQ, within the backward's
derived bounds (plus the 16-bit rounding of each dQ part).
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_19_amd.workloads import Workload, make_inputs
from oracle import attn_fwd_oracle
from parity_common import TOL_LSE, TOL_O, _check_full, _say, half_ulp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _w(B, Hq, Hkv, Sq, Sk, d, dt):
    return Workload(f"shard_b{B}_h{Hq}_{Hkv}_sq{Sq}_sk{Sk}_d{d}_{dt}", B, Hq, Hkv, Sq, Sk, d, dt,
                    True, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("kv_split", [1, 0, 3])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,cuts", [
    (1, 8, 2, 300, 1000, 128, "bf16", [0, 250, 640, 1000]),
    (2, 4, 4, 513, 513, 64, "f16", [0, 100, 300, 513]),
    (1, 16, 2, 700, 2100, 128, "bf16", [0, 1500, 2100]),
    (2, 32, 8, 1, 3000, 128, "bf16", [0, 1000, 2999, 3000]),   # decode kernel
    (1, 16, 4, 4, 1000, 64, "f16", [0, 500, 1000]),             # decode kernel
    (1, 8, 2, 300, 1000, 192, "bf16", [0, 250, 640, 1000]),     # 8-wave key halves
    (1, 6, 6, 200, 700, 176, "f16", [0, 333, 700]),             # padded 176 -> 192
])
def test_key_shards(B, Hq, Hkv, Sq, Sk, d, dt, cuts, kv_split):
    from exact_attention_19_amd import attn_fwd_causal_offset, attn_merge
    w = _w(B, Hq, Hkv, Sq, Sk, d, dt)
    q, k, v = make_inputs(w, seed=Sk + Sq)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        off = Sk - Sq - a
        _say(f"[gpu] attn_fwd_causal_offset {w.name} keys [{a}, {b}) offset {off} "
             f"kv_split={kv_split}")
        # k, v passed as strided slices of the full tensors
        o_p, l_p = attn_fwd_causal_offset(qg, kg[:, a:b], vg[:, a:b], off, scale=w.scale,
                                          kv_split=kv_split)
        torch.cuda.synchronize()
        ref = attn_fwd_oracle(q, k, v, w.scale, True, key_range=(a, b))
        _check_full(w, None, None, None, o_p.cpu(), l_p.cpu(), strict=False, ref=ref)
        outs.append(o_p)
        lses.append(l_p)
    o, lse = attn_merge(torch.stack(outs), torch.stack(lses), dtype=q.dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_fwd_oracle(q, k, v, w.scale, True)
    diff = np.abs(o.double().cpu().numpy() - o_ref)
    # the shard outputs were rounded to 16 bit before the merge
    bound = TOL_O[dt] + 2 * half_ulp(o_ref, dt)
    assert np.all(diff <= bound), f"max|dO| = {diff.max()}"
    fin = np.isfinite(lse_ref)
    lg = lse.double().cpu().numpy()
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= TOL_LSE


@pytest.mark.parametrize("Sq,Hq,Hkv", [(257, 8, 2), (1, 32, 8)])
def test_offset_sk_minus_sq_is_attn_fwd(Sq, Hq, Hkv):
    from exact_attention_19_amd import attn_fwd, attn_fwd_causal_offset
    w = _w(1, Hq, Hkv, Sq, 900, 128, "bf16")
    q, k, v = (t.cuda() for t in make_inputs(w, seed=3))
    o1, l1 = attn_fwd(q, k, v, scale=w.scale, causal=True)
    o2, l2 = attn_fwd_causal_offset(q, k, v, 900 - Sq, scale=w.scale, kv_split=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("Sq,Hq,Hkv", [(200, 4, 4), (2, 16, 4)])
def test_offsets_past_both_ends(Sq, Hq, Hkv):
    """An offset of Sk or more shows every key to every row (the non-causal
    result); one below -Sq + 1 shows none (O = 0, LSE = -inf)."""
    from exact_attention_19_amd import attn_fwd, attn_fwd_causal_offset
    w = _w(1, Hq, Hkv, Sq, 333, 64, "f16")
    q, k, v = (t.cuda() for t in make_inputs(w, seed=4))
    o_all, l_all = attn_fwd_causal_offset(q, k, v, 333, scale=w.scale)
    o_nc, l_nc = attn_fwd(q, k, v, scale=w.scale, causal=False)
    o_none, l_none = attn_fwd_causal_offset(q, k, v, -Sq, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.allclose(o_all.float(), o_nc.float(), atol=2e-3, rtol=0)
    assert torch.allclose(l_all, l_nc, atol=1e-4, rtol=0)
    assert torch.all(o_none == 0) and torch.all(torch.isneginf(l_none))


def _bwd_full(w, seed, fwd="oracle"):
    """Inputs, dO and the full problem's O and LSE on the GPU: the oracle's
    (rounded to the 16-bit type and fp32) or, fwd="gpu", the GPU forward's."""
    from exact_attention_19_amd import attn_fwd
    from test_bwd_gpu import oracle_forward
    q, k, v = make_inputs(w, seed=seed)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(seed + 1)).to(q.dtype)
    if fwd == "oracle":
        o, lse = (t.cuda() for t in oracle_forward(q, k, v, w))
    else:
        o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True)
    return q, k, v, do, o, lse


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,dt,cuts", [
    (1, 8, 2, 300, 1000, 128, "bf16", [0, 250, 640, 1000]),
    (2, 4, 4, 257, 257, 64, "f16", [0, 100, 257]),        # rows 0-99 see none of shard 2
    (1, 4, 1, 333, 200, 96, "bf16", [0, 64, 200]),        # rows with no key at all
    (2, 8, 4, 1, 700, 128, "bf16", [0, 300, 699, 700]),
])
def test_backward_key_shards(B, Hq, Hkv, Sq, Sk, d, dt, cuts):
    from exact_attention_19_amd import attn_bwd_causal_offset
    from oracle import attn_bwd_oracle
    from test_bwd_gpu import TINY, U, error_bounds
    w = _w(B, Hq, Hkv, Sq, Sk, d, dt)
    q, k, v, do, o, lse = _bwd_full(w, seed=Sq + Sk + d)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    rq, rk, rv = attn_bwd_oracle(q, k, v, do, w.scale, True)
    bq, bk, bv = error_bounds(q, k, v, do, o.cpu(), lse.cpu(), w.scale, True, dt)
    u = U[dt]
    dq_sum = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dq_mag = torch.zeros_like(dq_sum)
    for a, b in zip(cuts[:-1], cuts[1:]):
        off = Sk - Sq - a
        _say(f"[gpu] attn_bwd_causal_offset {w.name} keys [{a}, {b}) offset {off}")
        dq, dk, dv = attn_bwd_causal_offset(qg, kg[:, a:b].contiguous(), vg[:, a:b].contiguous(),
                                            o, lse, dog, off, scale=w.scale)
        torch.cuda.synchronize()
        for name, got, ref, bound in (("dk", dk, rk[:, a:b], bk[:, a:b]),
                                      ("dv", dv, rv[:, a:b], bv[:, a:b])):
            gd = got.double().cpu().numpy()
            allowed = 2.0 * (bound + u * np.abs(ref)) + 0.5 * TINY[dt]
            diff = np.abs(gd - ref)
            assert np.isfinite(gd).all() and np.all(diff <= allowed), \
                f"{name} [{a}, {b}): max|d| {diff.max():.3e}, worst use {(diff / allowed).max():.2f}"
        dq_sum += dq.float()
        dq_mag += dq.float().abs()
    gd = dq_sum.double().cpu().numpy()
    # each part was rounded to 16 bit once more than the single-call dQ
    allowed = 2.0 * (bq + u * np.abs(rq)) + u * dq_mag.double().cpu().numpy() \
        + len(cuts) * 0.5 * TINY[dt]
    diff = np.abs(gd - rq)
    assert np.all(diff <= allowed), \
        f"dq: max|d| {diff.max():.3e}, worst use {(diff / allowed).max():.2f}"


def test_backward_offset_sk_minus_sq_is_attn_bwd():
    from exact_attention_19_amd import attn_bwd, attn_bwd_causal_offset
    w = _w(1, 8, 2, 200, 333, 128, "bf16")
    q, k, v, do, o, lse = _bwd_full(w, seed=8)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    a = attn_bwd(qg, kg, vg, o, lse, dog, scale=w.scale, causal=True)
    b = attn_bwd_causal_offset(qg, kg, vg, o, lse, dog, 333 - 200, scale=w.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
