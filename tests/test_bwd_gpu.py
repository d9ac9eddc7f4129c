"""GPU parity of the backward pass (attn_bwd, through the C ABI) against the
fp64 oracle's gradients.

Inputs.  The backward consumes the forward's O and LSE.  The parity cases
feed it the oracle's O (rounded to the 16-bit type) and LSE (rounded to
fp32), so they test the backward kernels alone and their bound does not
depend on how accurate the GPU forward happens to be.  The composed cases
(GPU forward, then GPU backward, as a training step runs them) take the
forward's stated tolerances instead: |dLSE| <= 1e-3 and |dO| <= 2e-3 (fp16)
or 1e-2 (bf16) per element.

Bound.  No page fixes a precision for gradients, so each element's bound is
derived from the arithmetic (and written out below): with u the unit
roundoff of the 16-bit type (2^-8 bf16, 2^-11 fp16),
  P       is recomputed in fp32 from the given LSE: relative error
          e_P = e_LSE + 2^-20 (the error of the LSE handed in -- its fp32
          rounding, or the forward's tolerance -- plus exp2 and fp32
          rounding);
  D_i     = dO_i . O_i uses the given 16-bit O: |dD_i| = e_D,i +
          d 2^-24 |dO_i| . |O_i|, with e_D,i = |dO_i . (O_given - O)| for
          the rounded oracle O, or tol_O sum_c |dO_ic| for a forward within
          its tolerance;
  dS_ij   = P (dP - D), rounded to 16 bit once: |d dS| <= e_P |dS| +
          P |dD_i| + P d 2^-24 |dO_i| . |v_j| + u |dS| + t/2, with t the
          smallest spacing of the format (2^-24 for fp16, whose subnormals
          tiny dS and P values fall among);
  dV_j    = sum_i round16(P_ij) dO_i: |d dV_j| <= sum_i ((u + e_P) P_ij +
          t/2) |dO_i|;
  dQ, dK  = scale sums of the rounded dS times 16-bit K or Q:
          |d dQ_i| <= scale sum_j |d dS_ij| |k_j|, the same for dK;
plus fp32 accumulation (n 2^-24 of the sums of magnitudes) and the rounding
of the result to 16 bit (u |x|, and half the smallest spacing of the format
for results in the fp16 subnormal range).  The test allows twice that bound.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn_bwd_oracle, attn_fwd_oracle
from exact_attention_19_amd.workloads import WORKLOADS, Workload, make_inputs
from parity_common import TOL_LSE, TOL_O, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
TINY = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24}


def _f64(t):
    return t.detach().to("cpu").to(torch.float64)


def error_bounds(q, k, v, do, o_in, lse_in, scale, causal, dt, stated=False):
    """Elementwise bounds (dq, dk, dv) as derived in the module docstring,
    from fp64 quantities computed here with torch on the CPU.  o_in, lse_in:
    the O and LSE the backward was given.  stated=False: they are the
    oracle's, rounded, and their error is that rounding; stated=True: they
    come from the GPU forward, and only its stated tolerances are assumed."""
    u = U[dt]
    acc = 2.0 ** -24
    qd, kd, vd, dod, og = (_f64(t) for t in (q, k, v, do, o_in))
    B, Sq, Hq, d = qd.shape
    Sk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    qh = qd.permute(0, 2, 1, 3)                                   # (B, Hq, Sq, d)
    kh = kd.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)       # (B, Hq, Sk, d)
    vh = vd.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    doh = dod.permute(0, 2, 1, 3)
    s = torch.matmul(qh, kh.transpose(-1, -2)) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(j > i + (Sk - Sq), float("-inf"))
    m = s.amax(dim=-1, keepdim=True)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    e = torch.exp(s - m)
    z = e.sum(dim=-1, keepdim=True)
    p = torch.where(z > 0, e / torch.where(z > 0, z, torch.ones_like(z)), torch.zeros_like(e))
    lse_ref = torch.where(z[..., 0] > 0, m[..., 0] + torch.log(torch.where(z[..., 0] > 0, z[..., 0], torch.ones_like(z[..., 0]))),
                          torch.full_like(z[..., 0], float("-inf")))
    o = torch.matmul(p, vh)
    dp = torch.matmul(doh, vh.transpose(-1, -2))
    if stated:
        e_d = TOL_O[dt] * doh.abs().sum(-1)
    else:
        e_d = (doh * (og.permute(0, 2, 1, 3) - o)).sum(-1).abs()
    dD = e_d + d * acc * (doh.abs() * o.abs()).sum(-1)
    D = (p * dp).sum(-1)
    ds = p * (dp - D[..., None])
    fin = torch.isfinite(lse_ref)
    if stated:
        dl = TOL_LSE
    else:
        lg = _f64(lse_in)
        dl = (lg[fin] - lse_ref[fin]).abs().max().item() if fin.any() else 0.0
    # a relative error e^dl - 1 of P, about dl
    e_p = math.expm1(dl) + 2.0 ** -20
    dds = e_p * ds.abs() + p * dD[..., None] \
        + p * d * acc * torch.matmul(doh.abs(), vh.abs().transpose(-1, -2)) + u * ds.abs()
    # rounding to 16 bit: relative u, or half the smallest spacing where the
    # value falls among the fp16 subnormals
    dds = dds + acc * ds.abs() + 0.5 * TINY[dt]
    # dV: (B, Hq, Sk, d) summed over the query heads of each kv head
    bv = torch.matmul(p.transpose(-1, -2), doh.abs()) * (u + e_p + Sq * acc) \
        + 0.5 * TINY[dt] * doh.abs().sum(dim=-2, keepdim=True)
    bq = scale * torch.matmul(dds, kh.abs()) + scale * Sk * acc * torch.matmul(ds.abs(), kh.abs())
    bk = scale * torch.matmul(dds.transpose(-1, -2), qh.abs()) \
        + scale * Sq * acc * torch.matmul(ds.abs().transpose(-1, -2), qh.abs())
    bv = bv.reshape(B, Hkv, g, Sk, d).sum(2).permute(0, 2, 1, 3)
    bk = bk.reshape(B, Hkv, g, Sk, d).sum(2).permute(0, 2, 1, 3)
    bq = bq.permute(0, 2, 1, 3)
    return bq.numpy(), bk.numpy(), bv.numpy()


def oracle_forward(q, k, v, w):
    """The oracle's O rounded to the input type (RNE) and LSE rounded to fp32:
    the forward outputs the backward consumes, free of any GPU error."""
    o_ref, lse_ref = attn_fwd_oracle(q, k, v, w.scale, w.causal)
    return torch.from_numpy(o_ref).to(q.dtype), torch.from_numpy(lse_ref).to(torch.float32)


def _run(w: Workload, seed=0, dout_scale=1.0, fwd="oracle"):
    """fwd="oracle": the backward gets the oracle's O and LSE; fwd="gpu": the
    GPU forward's (the composed training step)."""
    from exact_attention_19_amd import attn_bwd, attn_fwd
    q, k, v = make_inputs(w, seed=seed)
    gen = torch.Generator().manual_seed(seed + 1000)
    do = (dout_scale * torch.randn(q.shape, generator=gen)).to(q.dtype)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    _say(f"[gpu] attn_bwd {w.name} B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} Hkv={w.Hkv} "
         f"d={w.d} {w.dtype} causal={w.causal} forward from the {fwd}")
    if fwd == "oracle":
        o, lse = (t.cuda() for t in oracle_forward(q, k, v, w))
    else:
        o, lse = attn_fwd(qg, kg, vg, scale=w.scale, causal=w.causal)
    dq, dk, dv = attn_bwd(qg, kg, vg, o, lse, dog, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return q, k, v, do, o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def _check(w, q, k, v, do, o, lse, dq, dk, dv, stated=False):
    rq, rk, rv = attn_bwd_oracle(q, k, v, do, w.scale, w.causal)
    bq, bk, bv = error_bounds(q, k, v, do, o, lse, w.scale, w.causal, w.dtype, stated=stated)
    u = U[w.dtype]
    worst = {}
    for name, got, ref, bound in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        gd = got.double().numpy()
        assert np.isfinite(gd).all(), f"{name} not finite"
        # + half the format's smallest spacing (fp16 subnormals: 2^-24)
        allowed = 2.0 * (bound + u * np.abs(ref)) + 0.5 * TINY[w.dtype]
        diff = np.abs(gd - ref)
        ratio = diff / allowed
        at = np.unravel_index(np.argmax(ratio), ratio.shape)
        worst[name] = (float(diff.max()), float(ratio.max()))
        assert np.all(diff <= allowed), (
            f"{w.name} {name}: |d| = {diff[at]:.3e} at {at} > bound {allowed[at]:.3e} "
            f"(ref {ref[at]:.4e}, got {gd[at]:.4e}); max|d| = {diff.max():.3e}")
    _say(f"{w.name}: " + ", ".join(f"{n} max|d| {a:.2e} (bound use {r:.2f})"
                                    for n, (a, r) in worst.items()))


def _cases():
    cases = []
    for dt in ("bf16", "f16"):
        cases += [
            Workload(f"bwd_mha_nc_{dt}", 1, 2, 2, 128, 128, 64, dt, False, 0.125),
            Workload(f"bwd_causal_sq_{dt}", 2, 4, 4, 257, 257, 128, dt, True, 1 / math.sqrt(128)),
            Workload(f"bwd_causal_off_{dt}", 1, 8, 2, 200, 333, 128, dt, True, 1 / math.sqrt(128)),
            Workload(f"bwd_causal_empty_rows_{dt}", 1, 4, 1, 333, 200, 64, dt, True, 0.2),
            Workload(f"bwd_gqa_nc_{dt}", 2, 8, 2, 190, 450, 128, dt, False, 1 / math.sqrt(128)),
        ]
    # head sizes 32 and 96 (one and three 32-column blocks)
    for d in (32, 96):
        cases += [
            Workload(f"bwd_d{d}_causal_off_bf16", 1, 8, 2, 200, 333, d, "bf16", True,
                     1 / math.sqrt(d)),
            Workload(f"bwd_d{d}_gqa_nc_f16", 2, 4, 1, 150, 270, d, "f16", False, 1 / math.sqrt(d)),
        ]
    cases += [Workload("bwd_scale1_f16", 1, 4, 4, 300, 300, 128, "f16", True, 1.0),
              Workload("bwd_one_row_bf16", 2, 8, 4, 1, 700, 128, "bf16", True, 1 / math.sqrt(128)),
              Workload("bwd_one_key_bf16", 1, 4, 2, 100, 1, 64, "bf16", False, 0.3)]
    return cases


@pytest.mark.parametrize("w", _cases(), ids=lambda w: w.name)
def test_bwd_parity(w):
    _check(w, *_run(w))


@pytest.mark.parametrize("w", [c for c in _cases() if c.name in (
    "bwd_causal_off_bf16", "bwd_causal_empty_rows_f16", "bwd_gqa_nc_bf16", "bwd_scale1_f16")],
    ids=lambda w: w.name)
def test_bwd_after_gpu_forward(w):
    """The training step as run: GPU forward, then GPU backward on its O and
    LSE, bounded with the forward's stated tolerances only."""
    _check(w, *_run(w, fwd="gpu"), stated=True)


def test_bwd_1k_causal_workload():
    """The 2 x 1024 causal fp16 MHA workload, every gradient element."""
    w = WORKLOADS["mha_causal_f16_b2_h16_s1024_d128"]
    _check(w, *_run(w))


def test_bwd_gqa_head_layout_at_1536():
    """The 8K GQA workload's heads (Hq 32, Hkv 8, d 128, bf16, causal) at
    1536 tokens: 12 key blocks of the dK/dV kernel, 24 query tiles per head,
    four query heads per kv head; every gradient element."""
    w = WORKLOADS["gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128"].with_(
        name="bwd_gqa4_bf16_s1536", Sq=1536, Sk=1536)
    _check(w, *_run(w))


@pytest.mark.timeout(900)
def test_bwd_full_size_kv_group():
    """The 8K GQA workload at full size, in the launch configuration that
    bench.py --backward times (all 32 query heads, 8 kv heads).  The
    gradients of kv group 0 (query heads 0-3, kv head 0) depend only on that
    group's tensors, so the oracle run on the group alone is their exact
    reference: every element of dq[:, :, 0:4], dk[:, :, 0] and dv[:, :, 0]."""
    from exact_attention_19_amd import attn_bwd, attn_fwd
    w = WORKLOADS["gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128"]
    g = w.Hq // w.Hkv
    sub = w.with_(name="bwd_gqa4_s8192_group0", Hq=g, Hkv=1)
    q, k, v = make_inputs(w, seed=0)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(1000)).to(q.dtype)
    hq = lambda t: t[:, :, :g].contiguous()
    hk = lambda t: t[:, :, :1].contiguous()
    # group 0's O and LSE from the oracle (on the group alone); the other
    # groups' from the GPU forward (they do not enter group 0's gradients)
    _say(f"[cpu] oracle forward of kv group 0 of {w.name}")
    o0, lse0 = oracle_forward(hq(q), hk(k), hk(v), sub)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    _say(f"[gpu] attn_fwd + attn_bwd {w.name}")
    o, lse = attn_fwd(qg, kg, vg, scale=w.scale, causal=w.causal)
    o[:, :, :g] = o0.cuda()
    lse[:, :g] = lse0.cuda()
    dq, dk, dv = attn_bwd(qg, kg, vg, o, lse, dog, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    _say(f"[cpu] oracle backward of kv group 0 of {w.name} (about half a minute)")
    _check(sub, hq(q), hk(k), hk(v), hq(do), o0, lse0, hq(dq), hk(dk), hk(dv))


def test_bwd_deterministic():
    from exact_attention_19_amd import attn_bwd, attn_fwd
    w = Workload("bwd_det", 1, 8, 2, 333, 517, 128, "bf16", True, 0.1)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=3))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(q.dtype).cuda()
    o, lse = attn_fwd(q, k, v, scale=w.scale, causal=True)
    a = attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True)
    b = attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_no_writes_outside_outputs():
    from exact_attention_19_amd import attn_bwd, attn_fwd
    w = Workload("bwd_canary", 1, 4, 2, 150, 170, 64, "f16", True, 0.2)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=5))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(6)).to(q.dtype).cuda()
    o, lse = attn_fwd(q, k, v, scale=w.scale, causal=True)
    pad = 4096
    bufs = []
    for ref in (q, k, v):
        n = ref.numel()
        buf = torch.full((n + 2 * pad,), 1234.0, dtype=ref.dtype, device="cuda")
        bufs.append((buf, buf[pad:pad + n].view(ref.shape), n))
    attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True,
             dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1])
    torch.cuda.synchronize()
    for buf, _, n in bufs:
        assert torch.all(buf[:pad] == 1234.0) and torch.all(buf[pad + n:] == 1234.0)


@pytest.mark.parametrize("w", [
    Workload("bwd_pad8_causal_off_bf16", 1, 8, 2, 200, 333, 8, "bf16", True, 1 / math.sqrt(8)),
    Workload("bwd_pad40_causal_off_f16", 1, 8, 2, 200, 333, 40, "f16", True, 1 / math.sqrt(40)),
    Workload("bwd_pad80_gqa_nc_bf16", 2, 8, 2, 190, 450, 80, "bf16", False, 1 / math.sqrt(80)),
    Workload("bwd_pad104_empty_rows_f16", 1, 4, 1, 333, 200, 104, "f16", True, 0.2),
    Workload("bwd_pad120_causal_bf16", 2, 4, 4, 257, 257, 120, "bf16", True, 1 / math.sqrt(120)),
], ids=lambda w: w.name)
def test_bwd_padded_head_sizes(w):
    """Head sizes that are multiples of 8 but not of 32 run on the kernels of
    the next built size: columns past d load as zeros and are not stored."""
    _check(w, *_run(w))


@pytest.mark.parametrize("w", [
    Workload("bwd_d192_causal_off_bf16", 1, 8, 2, 200, 333, 192, "bf16", True, 1 / math.sqrt(192)),
    Workload("bwd_d192_gqa_nc_f16", 2, 4, 1, 150, 270, 192, "f16", False, 1 / math.sqrt(192)),
    Workload("bwd_d256_causal_sq_f16", 2, 4, 4, 257, 257, 256, "f16", True, 1 / math.sqrt(256)),
    Workload("bwd_d256_causal_off_bf16", 1, 8, 2, 200, 333, 256, "bf16", True, 1 / math.sqrt(256)),
    Workload("bwd_d256_gqa_nc_bf16", 2, 8, 2, 190, 450, 256, "bf16", False, 1 / math.sqrt(256)),
    Workload("bwd_pad136_empty_rows_f16", 1, 4, 1, 333, 200, 136, "f16", True, 0.2),
    Workload("bwd_pad160_causal_off_f16", 1, 8, 2, 200, 333, 160, "f16", True, 1 / math.sqrt(160)),
    Workload("bwd_pad200_gqa_nc_bf16", 2, 4, 1, 150, 270, 200, "bf16", False, 1 / math.sqrt(200)),
    Workload("bwd_pad248_causal_bf16", 1, 4, 2, 300, 300, 248, "bf16", True, 1 / math.sqrt(248)),
    Workload("bwd_d256_one_row_f16", 1, 4, 2, 1, 700, 256, "f16", True, 1 / math.sqrt(256)),
    Workload("bwd_d192_one_key_bf16", 1, 4, 2, 100, 1, 192, "bf16", False, 0.3),
], ids=lambda w: w.name)
def test_bwd_large_head_sizes(w):
    """Head sizes above 128 run on the 192- and 256-column kernels, whose
    dK/dV workgroups hold 64 keys in 4 waves (and, at 256, one Q/dO buffer
    instead of two); d below the built size pads as for the smaller ones.
    Every case spans several 64-key blocks with a ragged last one."""
    _check(w, *_run(w))


@pytest.mark.parametrize("w", [
    Workload("bwd_d256_after_fwd_bf16", 1, 8, 2, 200, 333, 256, "bf16", True, 1 / math.sqrt(256)),
    Workload("bwd_pad200_after_fwd_f16", 1, 4, 4, 257, 257, 200, "f16", True, 1 / math.sqrt(200)),
], ids=lambda w: w.name)
def test_bwd_large_head_after_gpu_forward(w):
    """GPU forward, then GPU backward, at head sizes above 128."""
    _check(w, *_run(w, fwd="gpu"), stated=True)


def test_bwd_large_head_no_writes_outside_outputs():
    """d = 200 on the 256-column kernels: rows of the gradients are dense
    with 200 columns, so a column past d written by mistake would land on
    the next row or on a canary; every element between the canaries is
    written."""
    from exact_attention_19_amd import attn_bwd, attn_fwd
    w = Workload("bwd_canary_d200", 1, 4, 2, 150, 170, 200, "bf16", True, 0.1)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=7))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(8)).to(q.dtype).cuda()
    o, lse = attn_fwd(q, k, v, scale=w.scale, causal=True)
    pad = 4096
    bufs = []
    for ref in (q, k, v):
        n = ref.numel()
        buf = torch.full((n + 2 * pad,), 1234.0, dtype=ref.dtype, device="cuda")
        bufs.append((buf, buf[pad:pad + n].view(ref.shape), n))
    attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True,
             dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1])
    torch.cuda.synchronize()
    for buf, inner, n in bufs:
        assert torch.all(buf[:pad] == 1234.0) and torch.all(buf[pad + n:] == 1234.0)
        assert torch.all(inner != 1234.0)
