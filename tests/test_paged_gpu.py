"""GPU parity of decode over a paged K/V cache (attn_decode_paged), through the
C ABI, against the fp64 oracle (attn_decode_paged_oracle: each sequence's
keys gathered through its block table, then the dense forward).

The caches come from make_paged_cache: each sequence's blocks scattered over
a shuffled pool whose unused slots hold NaN, so a read of a wrong block, slot
or of a token past a sequence's length shows as a wrong or NaN output.
Sequences have ragged lengths (1, 15, 16, 17, 31, 32, 33, block multiples,
thousands, 0), the block sizes are 16 to 256 (16 and 48 put the two 16-key
halves of a 32-key tile in different blocks), and the key range is split or
not.
Tolerances as for the forward (2e-3 fp16, 1e-2 bf16 on O, with the half-ulp
allowance of the edge cases; 1e-3 on LSE).  Unsplit, a sequence's result is
also bit-for-bit the dense decode kernel's on its gathered keys.
"""
import math

import pytest
import torch

from exact_attention_19_amd.workloads import Workload, make_inputs, make_paged_cache
from parity_common import _check_full, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _run(name, lens, block_size, Hq=32, Hkv=8, Sq=1, d=128, dt="bf16", causal=True,
         kv_split=0, seed=0, max_seqlen=None, spare=3):
    from exact_attention_19_amd import attn_decode_paged
    from oracle import attn_decode_paged_oracle
    B = len(lens)
    S = max(max(lens), 1)
    w = Workload(name, B, Hq, Hkv, Sq, S, d, dt, causal, 1.0 / math.sqrt(d))
    q, k, v = make_inputs(w, seed=seed)
    need = sum(max(0, -(-L // block_size)) for L in lens)
    kp, vp, table, seqlens = make_paged_cache(k, v, lens, block_size,
                                              num_blocks=need + spare, seed=seed + 1)
    _say(f"[gpu] attn_decode_paged {name} lens={lens[:6]}{'...' if B > 6 else ''} "
         f"block={block_size} Hq={Hq} Hkv={Hkv} Sq={Sq} d={d} {dt} causal={causal} "
         f"kv_split={kv_split} max_seqlen={max_seqlen}")
    o, lse = attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), seqlens.cuda(),
                               scale=w.scale, causal=causal, kv_split=kv_split,
                               max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    ref = attn_decode_paged_oracle(q, kp, vp, table, seqlens, w.scale, causal,
                                   max_seqlen=max_seqlen)
    _check_full(w, None, None, None, o.cpu(), lse.cpu(), strict=False, ref=ref)
    return q, k, v, o, lse, w


@pytest.mark.parametrize("kv_split", [1, 0, 6])
@pytest.mark.parametrize("block_size", [16, 32, 48, 64, 256])
def test_paged_ragged_lengths(block_size, kv_split):
    lens = [1, 15, 16, 17, 31, 32, 33, 2 * block_size, 3000, 700, 4099]
    _run(f"paged_ragged_b{block_size}", lens, block_size, kv_split=kv_split, seed=block_size)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_paged_head_sizes_dtypes_masks(d, dt, causal):
    _run(f"paged_d{d}_{dt}_c{int(causal)}", [2000, 65, 1500], 64, Hq=16, Hkv=4, Sq=5, d=d,
         dt=dt, causal=causal, kv_split=0, seed=d + int(causal))


@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("Hq,Hkv,Sq", [(32, 8, 4), (8, 1, 4), (4, 4, 8), (1, 1, 32),
                                       (12, 3, 3), (64, 4, 4), (32, 2, 6)])
def test_paged_group_sizes_and_tokens(Hq, Hkv, Sq, block_size):
    # lengths shorter than Sq: the first rows see no key (O = 0, LSE = -inf)
    _run(f"paged_g{Hq // Hkv}_sq{Sq}", [2, 1, 999, 32, 18], block_size, Hq=Hq, Hkv=Hkv, Sq=Sq,
         kv_split=3, seed=Hq + Sq)


@pytest.mark.parametrize("kv_split", [1, 0, 4])
def test_paged_empty_sequences(kv_split):
    _run("paged_empty", [0, 500, 0, 64], 64, kv_split=kv_split, seed=5)


def test_paged_max_seqlen_bounds_lengths():
    """Lengths above max_seqlen are taken as max_seqlen (the oracle clamps
    the same way); max_seqlen also sizes the key split."""
    _run("paged_clamp", [5000, 300, 2048], 64, kv_split=0, seed=6, max_seqlen=2048)


@pytest.mark.parametrize("block_size", [16, 64])
def test_paged_unsplit_equals_dense_decode_bit_for_bit(block_size):
    from exact_attention_19_amd import attn_fwd_split
    lens = [777, 64, 2049, 17]
    q, k, v, o, lse, w = _run("paged_vs_dense", lens, block_size, kv_split=1, seed=7)
    for b, L in enumerate(lens):
        od, ld = attn_fwd_split(q[b:b + 1].cuda(), k[b:b + 1, :L].contiguous().cuda(),
                                v[b:b + 1, :L].contiguous().cuda(), scale=w.scale,
                                causal=True, kv_split=1)
        torch.cuda.synchronize()
        assert torch.equal(od[0].cpu(), o[b].cpu()), b
        assert torch.equal(ld[0].cpu(), lse[b].cpu()), b


def test_paged_bench_shape_full_compare():
    """32 sequences of 4K-8K keys, block 64, the 8K GQA heads: every output
    element against the oracle, in the launch configuration bench.py times."""
    g = torch.Generator().manual_seed(11)
    lens = torch.randint(4096, 8193, (32,), generator=g).tolist()
    _run("paged_b32_gqa4_sk8k", lens, 64, kv_split=0, seed=11, max_seqlen=8192)


def test_paged_rejects_mismatched_tensors():
    from exact_attention_19_amd import attn_decode_paged
    q = torch.zeros(2, 1, 8, 128, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(4, 32, 2, 128, dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    n = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        attn_decode_paged(q, kp, kp, t.long(), n)
    with pytest.raises(ValueError):
        attn_decode_paged(q, kp, kp, t[:1], n)
    with pytest.raises(ValueError):
        attn_decode_paged(q, kp, kp[:, :, :1], t, n)
