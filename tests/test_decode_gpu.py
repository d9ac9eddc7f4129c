"""GPU parity of the decode kernel (shapes whose query rows per kv head,
Hq / Hkv * Sq, number at most 32, or at most 128 in 32-row groups when
Sq <= 8, at d = 32, 64, 96 or 128), through the C ABI,
against the fp64 oracle: every output element, whole and with the key range
cut into pieces over workgroups, across GQA group sizes, token counts, causal
offsets, ragged key lengths and strided inputs.  Tolerances as for the
forward (2e-3 fp16, 1e-2 bf16 on O, with the half-ulp allowance for large
outputs of the edge shapes; 1e-3 on LSE).
"""
import math

import pytest
import torch

from exact_attention_19_amd.binding import ATTN_DTYPE_BF16, ATTN_DTYPE_F16
from exact_attention_19_amd.workloads import Workload, make_inputs
from parity_common import _check_full, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _cases():
    out = []
    for (Hq, Hkv, Sq) in ((32, 8, 1), (32, 8, 4), (8, 1, 4), (16, 2, 2), (4, 4, 8),
                          (2, 1, 16), (1, 1, 32), (8, 8, 1), (12, 3, 3)):
        for Sk in (1, 31, 33, 700, 4099):
            out.append((Hq, Hkv, Sq, Sk, 128, "bf16", True))
    for d in (64, 128):
        for dt in ("f16", "bf16"):
            for causal in (False, True):
                out.append((16, 4, 5, 2000, d, dt, causal))
    # more than 32 rows per kv head (Sq <= 8): 32-row groups, one workgroup
    # each; the last group partly filled (96 = 3 x 32 + 0, 40 = 32 + 8, ...)
    for (Hq, Hkv, Sq) in ((64, 4, 4), (32, 4, 8), (64, 2, 3), (40, 4, 4), (128, 8, 8)):
        for Sk in (1, 33, 4099):
            out.append((Hq, Hkv, Sq, Sk, 128, "bf16", True))
    for d in (64, 128):
        out.append((48, 2, 2, 1500, d, "f16", False))
    # head sizes 32 and 96 (one and three 32-column blocks; the merge area's
    # swizzle stays inside rows that are not a multiple of 64 columns)
    for d in (32, 96):
        for dt in ("f16", "bf16"):
            out.append((32, 8, 2, 2049, d, dt, True))
            out.append((64, 4, 4, 700, d, dt, False))
    return out


@pytest.mark.parametrize("kv_split", [1, 0, 7])
@pytest.mark.parametrize("Hq,Hkv,Sq,Sk,d,dt,causal", _cases())
def test_decode_kernel(Hq, Hkv, Sq, Sk, d, dt, causal, kv_split):
    from exact_attention_19_amd import attn_fwd_plan, attn_fwd_split
    w = Workload(f"dec_h{Hq}_{Hkv}_sq{Sq}_sk{Sk}_d{d}_{dt}_c{int(causal)}", 2, Hq, Hkv, Sq, Sk,
                 d, dt, causal, 1.0 / math.sqrt(d))
    code = ATTN_DTYPE_BF16 if dt == "bf16" else ATTN_DTYPE_F16
    assert attn_fwd_plan(2, Sq, Sk, Hq, Hkv, d, int(causal), code)["decode"] == 1
    q, k, v = make_inputs(w, seed=Sk + 31 * Sq)
    _say(f"[gpu] decode {w.name} kv_split={kv_split}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=causal,
                            kv_split=kv_split)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_decode_attn_fwd_without_workspace():
    """attn_fwd (no workspace) runs the decode kernel unsplit."""
    from exact_attention_19_amd import attn_fwd
    w = Workload("dec_fwd", 3, 32, 8, 2, 5000, 128, "bf16", True, 1.0 / math.sqrt(128))
    q, k, v = make_inputs(w, seed=1)
    o, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


@pytest.mark.parametrize("kv_split", [1, 0])
def test_decode_strided_bhsd_and_packed(kv_split):
    """Decode on (B, H, S, d) views and on q, k, v sliced from one packed
    projection."""
    from exact_attention_19_amd import attn_fwd_strided
    w = Workload("dec_bhsd", 2, 16, 4, 3, 1500, 128, "f16", True, 1.0 / math.sqrt(128))
    q, k, v = make_inputs(w, seed=2)
    qh, kh, vh = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
    o, lse = attn_fwd_strided(qh, kh, vh, scale=w.scale, causal=True, layout="bhsd",
                              kv_split=kv_split)
    torch.cuda.synchronize()
    _check_full(w, q, k, v, o.transpose(1, 2).cpu(), lse.cpu(), strict=False)
    w2 = Workload("dec_packed", 2, 8, 2, 4, 4, 128, "bf16", False, 0.1)
    q2, k2, v2 = make_inputs(w2, seed=3)
    packed = torch.cat([q2, k2, v2], dim=2).cuda()
    o2, l2 = attn_fwd_strided(packed[:, :, :8], packed[:, :, 8:10], packed[:, :, 10:],
                              scale=w2.scale, causal=False, kv_split=kv_split)
    torch.cuda.synchronize()
    _check_full(w2, q2, k2, v2, o2.cpu(), l2.cpu(), strict=False)


def test_decode_deterministic_and_no_stray_writes():
    from exact_attention_19_amd import attn_fwd_split
    w = Workload("dec_canary", 1, 32, 8, 1, 3000, 128, "bf16", True, 0.1)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=5))
    n_o = w.B * w.Sq * w.Hq * w.d
    pad = 4096
    obuf = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((w.B * w.Hq * w.Sq + 2 * pad,), 777.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n_o].view(w.B, w.Sq, w.Hq, w.d)
    lse = lbuf[pad:pad + w.B * w.Hq * w.Sq].view(w.B, w.Hq, w.Sq)
    attn_fwd_split(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    o1, l1 = o.clone(), lse.clone()
    attn_fwd_split(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n_o:] == 1234.0)
    assert torch.all(lbuf[:pad] == 777.0) and torch.all(lbuf[-pad:] == 777.0)
    assert torch.equal(o, o1) and torch.equal(lse, l1)
