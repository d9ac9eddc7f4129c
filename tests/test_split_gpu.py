"""GPU parity of the key split (attn_fwd_split) and of the merge of partial
states (attn_merge), through the C ABI, against the fp64 oracle.

attn_fwd_split must give the attention of attn_fwd to the same tolerances
(2e-3 fp16, 1e-2 bf16 on O; 1e-3 on LSE), for every split count, including
pieces that see no key of a row and rows that see no key at all.  attn_merge
is checked against the oracle's merge of the same partial states, and, as the
one-device half of a key-sharded (context-parallel) attention, on attn_fwd
outputs over key shards.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn_fwd_oracle, merge_partials_oracle
from exact_attention_19_amd.workloads import WORKLOADS, Workload, make_inputs
from parity_common import TOL_LSE, TOL_O, _check_full, _say, half_ulp

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


def _run_split(q, k, v, w: Workload, kv_split, workspace=None):
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan
    plan = attn_fwd_split_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d, int(w.causal),
                               _code(w.dtype), kv_split)
    _say(f"[gpu] attn_fwd_split {w.name} B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} "
         f"Hkv={w.Hkv} d={w.d} {w.dtype} causal={w.causal} kv_split={kv_split} {plan}")
    o, lse = attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=w.causal,
                            kv_split=kv_split, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), plan


SMALL = ["mha_tiny_f16_b1_h2_s128_d64",
         "mha_causal_f16_b2_h16_s1024_d128",
         "mha_causal_offset_f16_b1_h16_sq1280_sk1536_d128",
         "mha_causal_ragged_f16_b1_h16_sq1237_sk1531_d128"]


_REF = {}


def _oracle_of(name):
    """Inputs and oracle result of a named workload (computed once)."""
    if name not in _REF:
        w = WORKLOADS[name]
        q, k, v = make_inputs(w, seed=0)
        _REF[name] = (q, k, v, attn_fwd_oracle(q, k, v, w.scale, w.causal))
    return _REF[name]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("kv_split", [0, 2, 3, 64])
def test_split_small_workloads_full_parity(name, kv_split):
    w = WORKLOADS[name]
    q, k, v, ref = _oracle_of(name)
    o, lse, plan = _run_split(q, k, v, w, kv_split)
    err = _check_full(w, q, k, v, o, lse, ref=ref)
    _say(f"{name} split {kv_split} ({plan['pieces']} pieces): max|dO| = {err:.3e}")


def _split_edge_cases():
    cases = []
    # ragged lengths, both offsets, rows with no key (Sq > Sk, causal),
    # pieces that see none of a row's keys, GQA groups, both head sizes
    for Sq, Sk in ((300, 300), (129, 700), (700, 129), (513, 1000), (1000, 513),
                   (64, 2000), (1, 1500), (333, 65)):
        for causal in (False, True):
            cases.append((Sq, Sk, causal, 128, "bf16", 8, 2))
    for d in (64, 128):
        for dt in ("f16", "bf16"):
            cases.append((450, 777, True, d, dt, 4, 4))
            cases.append((777, 450, True, d, dt, 8, 1))
    return cases


@pytest.mark.parametrize("kv_split", [2, 5, 1000])
@pytest.mark.parametrize("Sq,Sk,causal,d,dt,Hq,Hkv", _split_edge_cases())
def test_split_edges(Sq, Sk, causal, d, dt, Hq, Hkv, kv_split):
    w = Workload(f"split_sq{Sq}_sk{Sk}_c{int(causal)}_d{d}_{dt}_h{Hq}_{Hkv}", 2, Hq, Hkv,
                 Sq, Sk, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=Sq * 7 + Sk)
    o, lse, _ = _run_split(q, k, v, w, kv_split)
    _check_full(w, q, k, v, o, lse, strict=False)


def test_split_one_is_attn_fwd_bit_for_bit():
    from exact_attention_19_amd import attn_fwd
    w = WORKLOADS["mha_causal_offset_f16_b1_h16_sq1280_sk1536_d128"]
    q, k, v = make_inputs(w, seed=2)
    o1, l1, plan = _run_split(q, k, v, w, 1)
    assert plan["keys_per_piece"] == 0
    o2, l2 = attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.cpu()) and torch.equal(l1, l2.cpu())


def test_split_workspace_contents_do_not_matter_and_reuse():
    """A workspace full of NaN, then reused by a second, smaller problem."""
    from exact_attention_19_amd import attn_fwd_split_workspace
    w1 = WORKLOADS["mha_causal_f16_b2_h16_s1024_d128"]
    w2 = Workload("reuse_small", 1, 4, 2, 700, 900, 64, "f16", True, 0.2)
    n1 = attn_fwd_split_workspace(w1.B, w1.Sq, w1.Sk, w1.Hq, w1.Hkv, w1.d, 1, _code("f16"), 3)
    n2 = attn_fwd_split_workspace(w2.B, w2.Sq, w2.Sk, w2.Hq, w2.Hkv, w2.d, 1, _code("f16"), 3)
    assert 0 < n2 < n1
    ws = torch.full((n1 // 4 + 64,), float("nan"), dtype=torch.float32,
                    device="cuda").view(torch.uint8)
    for w in (w1, w2):
        q, k, v = make_inputs(w, seed=4)
        o, lse, _ = _run_split(q, k, v, w, 3, workspace=ws)
        _check_full(w, q, k, v, o, lse, strict=w is w1)


@pytest.mark.parametrize("kv_split", [2, 0])
def test_split_graph_replays(kv_split):
    """A forward call captured in a HIP graph: every replay gives the eager
    result, with eager split calls of another shape reusing the same
    workspace between the replays.  kv_split = 2: the attention kernel writes
    two pieces' states and the merge kernel combines them; 0: the library's
    choice, here the unsplit key halves (one launch, the two halves' states
    merged in LDS)."""
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_plan, attn_fwd_split_workspace
    w = WORKLOADS["mha_causal_offset_f16_b1_h16_sq1280_sk1536_d128"]
    plan = attn_fwd_split_plan(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d, 1, _code("f16"), kv_split)
    assert plan["pieces"] == (2 if kv_split == 2 else 1), plan
    assert plan["key_halves"] == (1 if kv_split == 0 else 0), plan
    q, k, v = (t.cuda() for t in make_inputs(w, seed=0))
    w2 = Workload("graph_other", 1, 4, 2, 700, 900, 64, "f16", True, 0.2)
    q2, k2, v2 = (t.cuda() for t in make_inputs(w2, seed=3))
    n = max(attn_fwd_split_workspace(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d, 1, _code("f16"),
                                     kv_split),
            attn_fwd_split_workspace(w2.B, w2.Sq, w2.Sk, w2.Hq, w2.Hkv, w2.d, 1, _code("f16"), 3))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=kv_split,
                                  workspace=ws)
    o2_ref, l2_ref = attn_fwd_split(q2, k2, v2, scale=w2.scale, causal=True, kv_split=3,
                                    workspace=ws)
    out = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=kv_split, out=out,
                       lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=kv_split, out=out,
                       lse=lse, workspace=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say(f"[gpu] graph replay {rep}")
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), rep
        o2, l2 = attn_fwd_split(q2, k2, v2, scale=w2.scale, causal=True, kv_split=3,
                                workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, o2_ref) and torch.equal(l2, l2_ref), rep


def test_split_rejects_small_workspace():
    from exact_attention_19_amd import AttnError, attn_fwd_split
    w = WORKLOADS["mha_causal_f16_b2_h16_s1024_d128"]
    q, k, v = (t.cuda() for t in make_inputs(w, seed=0))
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(AttnError):
        attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=4, workspace=ws)


def test_split_no_writes_outside_outputs():
    from exact_attention_19_amd import attn_fwd_split
    w = Workload("split_canary", 1, 8, 2, 333, 650, 128, "bf16", True, 0.1)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=5))
    n_o = w.B * w.Sq * w.Hq * w.d
    pad = 4096
    obuf = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    n_l = w.B * w.Hq * w.Sq
    lbuf = torch.full((n_l + 2 * pad,), 777.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n_o].view(w.B, w.Sq, w.Hq, w.d)
    lse = lbuf[pad:pad + n_l].view(w.B, w.Hq, w.Sq)
    attn_fwd_split(q, k, v, scale=w.scale, causal=True, kv_split=4, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n_o:] == 1234.0)
    assert torch.all(lbuf[:pad] == 777.0) and torch.all(lbuf[pad + n_l:] == 777.0)
    assert torch.all(lse != 777.0)


def test_split_deterministic():
    from exact_attention_19_amd import attn_fwd_split
    w = WORKLOADS["mha_causal_f16_b2_h16_s1024_d128"]
    q, k, v = (t.cuda() for t in make_inputs(w, seed=1))
    o1, l1 = attn_fwd_split(q, k, v, scale=w.scale, causal=True)
    o2, l2 = attn_fwd_split(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_full_size_gqa_sampled_rows():
    """The 8K GQA workload forced into two pieces per block: sampled rows."""
    w = WORKLOADS["gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128"]
    q, k, v = make_inputs(w, seed=0)
    o, lse, plan = _run_split(q, k, v, w, 2)
    assert plan["pieces"] == 2
    r = np.random.default_rng(3)
    rows = []
    for h in (0, 5, 31):
        pick = {0, 1, 4095, 4096, 4097, 8190, 8191} | set(r.integers(0, w.Sq, 8).tolist())
        rows += [(h * w.Sq) + i for i in sorted(pick)]
    rows = np.array(rows, dtype=np.int64)
    o_ref, lse_ref = attn_fwd_oracle(q, k, v, w.scale, w.causal, rows=rows)
    i, h = rows % w.Sq, rows // w.Sq
    err = np.abs(o.double().numpy()[0, i, h] - o_ref).max()
    el = np.abs(lse.double().numpy()[0, h, i] - lse_ref).max()
    _say(f"split 8K GQA sampled: max|dO| = {err:.3e}, max|dLSE| = {el:.3e}")
    assert err <= TOL_O["bf16"] and el <= TOL_LSE


# ------------------------------------------------------------------ merge

def _oracle_parts(q, k, v, scale, causal, cuts):
    parts = [attn_fwd_oracle(q, k, v, scale, causal, key_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


@pytest.mark.parametrize("parts_dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_matches_oracle_merge(parts_dt, d):
    """attn_merge on partial states (rounded to the parts' dtype) against the
    oracle's fp64 merge of exactly those rounded states."""
    from exact_attention_19_amd import attn_merge
    B, Sq, Sk, Hq, Hkv = 2, 150, 400, 4, 2
    w = Workload("merge_parts", B, Hq, Hkv, Sq, Sk, d, "f16", True, 0.3)
    q, k, v = make_inputs(w, seed=d)
    cuts = [0, 37, 100, 101, 250, 400]  # includes a single-key range
    op, lp = _oracle_parts(q, k, v, w.scale, True, cuts)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[parts_dt]
    op_t = torch.from_numpy(op).to(tdt)
    lp_t = torch.from_numpy(lp).to(torch.float32)
    o_ref, lse_ref = merge_partials_oracle(op_t.double().numpy(), lp_t.double().numpy())
    for out_dt in ("f16", "bf16"):
        odt = torch.float16 if out_dt == "f16" else torch.bfloat16
        _say(f"[gpu] attn_merge parts={parts_dt} d={d} out={out_dt} P={len(cuts) - 1}")
        o, lse = attn_merge(op_t.cuda(), lp_t.cuda(), dtype=odt)
        torch.cuda.synchronize()
        diff = np.abs(o.double().cpu().numpy() - o_ref)
        # fp32 arithmetic, then one rounding to the output format
        bound = half_ulp(o_ref, out_dt) + 1e-5
        assert np.all(diff <= bound), f"max|dO| = {diff.max()}"
        lg = lse.double().cpu().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-5 * (1 + np.abs(lse_ref[fin]).max())


def test_merge_empty_parts_and_rows():
    """Parts with lse = -inf carry no weight; rows no part saw give 0, -inf."""
    from exact_attention_19_amd import attn_merge
    P, B, Sq, Hq, d = 3, 1, 40, 2, 64
    r = np.random.default_rng(9)
    op = r.standard_normal((P, B, Sq, Hq, d)).astype(np.float32)
    lp = r.standard_normal((P, B, Hq, Sq)).astype(np.float32)
    lp[1] = -np.inf                    # part 1 saw nothing
    op[1] = 0.0
    lp[:, :, :, :5] = -np.inf          # rows 0..4 seen by no part
    op[:, :, :5] = 0.0
    o_ref, lse_ref = merge_partials_oracle(op.astype(np.float64), lp.astype(np.float64))
    o, lse = attn_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(),
                        dtype=torch.bfloat16)
    torch.cuda.synchronize()
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(og[:, :5] == 0) and np.all(np.isneginf(lg[:, :, :5]))
    assert np.all(np.abs(og - o_ref) <= half_ulp(o_ref, "bf16") + 1e-5)
    fin = np.isfinite(lse_ref)
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-5


@pytest.mark.parametrize("P", [1, 2, 3, 7, 9, 16, 17, 37])
def test_merge_many_parts(P):
    """Part counts on both sides of the merge's batch sizes (2, 4, 8, 16),
    with LSEs growing by part (each batch raises the running max, so the sums
    are rescaled), the first parts empty for some rows (the max starts at
    -inf), and rows no part saw, against the fp64 oracle merge."""
    from exact_attention_19_amd import attn_merge
    B, Sq, Hq, d = 1, 24, 2, 128
    r = np.random.default_rng(100 + P)
    op = r.standard_normal((P, B, Sq, Hq, d)).astype(np.float32)
    lp = (np.arange(P, dtype=np.float32)[:, None, None, None] * 1.5
          + r.standard_normal((P, B, Hq, Sq)).astype(np.float32))
    lp[: P // 2, :, :, 5:10] = -np.inf     # rows 5..9: the first half of the parts saw nothing
    op[: P // 2, :, 5:10] = 0.0
    lp[:, :, :, :3] = -np.inf              # rows 0..2: no part saw anything
    op[:, :, :3] = 0.0
    o_ref, lse_ref = merge_partials_oracle(op.astype(np.float64), lp.astype(np.float64))
    _say(f"[gpu] attn_merge P={P} d={d}")
    o, lse = attn_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(),
                        dtype=torch.bfloat16)
    torch.cuda.synchronize()
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(og[:, :3] == 0) and np.all(np.isneginf(lg[:, :, :3]))
    assert np.all(np.abs(og - o_ref) <= half_ulp(o_ref, "bf16") + 1e-5), np.abs(og - o_ref).max()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.abs(lg[fin] - lse_ref[fin]).max() <= 1e-5 * (1 + np.abs(lse_ref[fin]).max())


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_key_shards_merged_equal_full_attention(dt):
    """Key-sharded attention on one device: attn_fwd on each key shard (no
    mask), attn_merge of the 16-bit shard outputs and their LSE; the result
    is the attention over all keys, within the tolerance plus the extra
    rounding of the shard outputs."""
    from exact_attention_19_amd import attn_fwd, attn_merge
    w = Workload("shards", 1, 8, 2, 300, 1000, 128, dt, False, 1.0 / math.sqrt(128))
    q, k, v = make_inputs(w, seed=11)
    cuts = [0, 250, 640, 1000]
    qg = q.cuda()
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o_p, l_p = attn_fwd(qg, k[:, a:b].contiguous().cuda(), v[:, a:b].contiguous().cuda(),
                            scale=w.scale, causal=False)
        outs.append(o_p)
        lses.append(l_p)
    o, lse = attn_merge(torch.stack(outs), torch.stack(lses), dtype=q.dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = attn_fwd_oracle(q, k, v, w.scale, False)
    diff = np.abs(o.double().cpu().numpy() - o_ref)
    bound = TOL_O[dt] + half_ulp(o_ref, dt)
    assert np.all(diff <= bound), f"max|dO| = {diff.max()}"
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= TOL_LSE


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("kv_split", [0, 1, 8])
@pytest.mark.parametrize("name", ["decode_gqa4_bf16_b32_hq32_hkv8_sq1_sk8192_d128",
                                  "decode_gqa4_bf16_b1_hq32_hkv8_sq1_sk32768_d128",
                                  "decode_gqa4_bf16_b32_hq32_hkv8_sq4_sk8192_d128"])
def test_decode_workloads_full_parity(name, kv_split):
    """Decode (one or four new tokens per sequence over a long K/V cache) at
    full size, every output row against the oracle, whole and split."""
    w = WORKLOADS[name]
    q, k, v, ref = _oracle_of(name)
    o, lse, plan = _run_split(q, k, v, w, kv_split)
    err = _check_full(w, q, k, v, o, lse, ref=ref)
    _say(f"{name} split {kv_split} ({plan['pieces']} pieces): max|dO| = {err:.3e}")
