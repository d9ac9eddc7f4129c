"""Seeded synthetic inputs for the attention forward.

This module only draws random numbers; it holds none of attention's
arithmetic.  Both the GPU path's tests and the oracle's tests take their inputs
from here, so the two sides see identical bytes.

Recipe (the same for every workload): one CPU ``torch.Generator`` seeded with
``seed`` (default 0) draws fp32 values in the order Q, K, V, then the outlier
rows; the fp32 values are then rounded to the workload's dtype (round to
nearest even).  Distributions:

* ``normal``:  Q, K, V ~ N(0, 1).
* ``outlier``: Q ~ N(0, 1); K ~ N(0, 1) with round(0.01 * Sk) distinct key
  rows per (batch, kv head), picked by ``randperm``, multiplied by 8 (exact in
  bf16); V ~ U(-1, 1) drawn as 2 * rand - 1.  Large scores from the scaled
  rows exercise the running-max rescaling of online softmax.

The shapes follow the pages' workloads: a tiny MHA case, the p1/p3-style
1K-2K causal MHA shapes (the CuTe DSL Ampere example's Sq=1280, Sk=1536,
H=16, d=128, scale 1.0 case), and Qwen3-like GQA prefill layouts at 8K and
16K (the MiniPaged-Qwen page's GQA head grouping), and decode: one (or a
few) new query tokens per sequence over a long cached K/V, the phase the
MiniPaged-Qwen page (section 19) sets apart from prefill because the query
side then has almost no parallelism and the work becomes reading the K/V
cache.  Layout is (batch, seq, heads, d_head).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    scale: float
    dist: str = "normal"

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def offset(self) -> int:
        """Bottom-right causal offset: query i sees keys j <= i + offset."""
        return self.Sk - self.Sq

    def metric_flops(self) -> float:
        """4*Sq*Sk*d*Hq*B, halved when causal (the headline FLOP convention)."""
        f = 4.0 * self.Sq * self.Sk * self.d * self.Hq * self.B
        return f / 2 if self.causal else f

    def visible_pairs(self) -> int:
        """Exact number of (query, key) pairs the mask lets through, per
        (batch, query head)."""
        if not self.causal:
            return self.Sq * self.Sk
        total = 0
        off = self.offset
        # row i sees min(Sk, max(0, i + off + 1)) keys
        for i in range(self.Sq):
            total += min(self.Sk, max(0, i + off + 1))
        return total

    def exact_flops(self) -> float:
        return 4.0 * self.d * self.visible_pairs() * self.Hq * self.B

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once (2 bytes/element), LSE fp32."""
        q = self.B * self.Sq * self.Hq * self.d * 2
        kv = self.B * self.Sk * self.Hkv * self.d * 2
        lse = self.B * self.Hq * self.Sq * 4
        return 2 * q + 2 * kv + lse

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("mha_tiny_f16_b1_h2_s128_d64", 1, 2, 2, 128, 128, 64, "f16",
                 False, 1.0 / 8.0),
        Workload("mha_causal_f16_b2_h16_s1024_d128", 2, 16, 16, 1024, 1024,
                 128, "f16", True, 1.0 / math.sqrt(128)),
        Workload("mha_causal_offset_f16_b1_h16_sq1280_sk1536_d128", 1, 16, 16,
                 1280, 1536, 128, "f16", True, 1.0),
        Workload("mha_causal_ragged_f16_b1_h16_sq1237_sk1531_d128", 1, 16, 16,
                 1237, 1531, 128, "f16", True, 1.0),
        Workload("gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128", 1, 32, 8, 8192,
                 8192, 128, "bf16", True, 1.0 / math.sqrt(128)),
        Workload("gqa8_causal_outlier_bf16_b1_hq32_hkv4_s16384_d128", 1, 32, 4,
                 16384, 16384, 128, "bf16", True, 1.0 / math.sqrt(128),
                 "outlier"),
        # the MiniPaged-Qwen page's Qwen3-0.6B attention heads (Hq 16, Hkv 8,
        # group 2, d 128) on 4K-token prompts, 4 sequences
        Workload("gqa2_causal_bf16_b4_hq16_hkv8_s4096_d128", 4, 16, 8, 4096, 4096, 128, "bf16",
                 True, 1.0 / math.sqrt(128)),
        # decode: the 8K GQA heads, one new token for each of 32 sequences
        Workload("decode_gqa4_bf16_b32_hq32_hkv8_sq1_sk8192_d128", 32, 32, 8, 1,
                 8192, 128, "bf16", True, 1.0 / math.sqrt(128)),
        # decode of one long sequence: only the key split fills the GPU
        Workload("decode_gqa4_bf16_b1_hq32_hkv8_sq1_sk32768_d128", 1, 32, 8, 1,
                 32768, 128, "bf16", True, 1.0 / math.sqrt(128)),
        # four new tokens per sequence (bottom-right causal among themselves)
        Workload("decode_gqa4_bf16_b32_hq32_hkv8_sq4_sk8192_d128", 32, 32, 8, 4,
                 8192, 128, "bf16", True, 1.0 / math.sqrt(128)),
    ]
}

# The workload the throughput figure is quoted on.
HEADLINE = "gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128"
# The largest single-GPU workload.
LARGEST = "gqa8_causal_outlier_bf16_b1_hq32_hkv4_s16384_d128"
# Decode workloads (bound by reading K and V from HBM).
DECODE = [n for n in WORKLOADS if n.startswith("decode_")]


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """Draw (q, k, v) for workload ``w`` following the module's recipe.

    Returns tensors of dtype ``DTYPES[w.dtype]`` on ``device``; q is
    (B, Sq, Hq, d), k and v are (B, Sk, Hkv, d)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    qs = (w.B, w.Sq, w.Hq, w.d)
    ks = (w.B, w.Sk, w.Hkv, w.d)
    q = torch.randn(qs, generator=g, dtype=torch.float32)
    k = torch.randn(ks, generator=g, dtype=torch.float32)
    if w.dist == "normal":
        v = torch.randn(ks, generator=g, dtype=torch.float32)
    elif w.dist == "outlier":
        v = 2.0 * torch.rand(ks, generator=g, dtype=torch.float32) - 1.0
        n_out = int(round(0.01 * w.Sk))
        for b in range(w.B):
            for h in range(w.Hkv):
                idx = torch.randperm(w.Sk, generator=g)[:n_out]
                k[b, idx, h, :] *= 8.0
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    dt = DTYPES[w.dtype]
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if str(device) != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def input_digest(q, k, v) -> str:
    """SHA-256 over the raw bytes of q, k, v (in that order)."""
    h = hashlib.sha256()
    for t in (q, k, v):
        t = t.detach().to("cpu").contiguous()
        h.update(t.view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def small_integer_inputs(w: Workload, seed: int = 0, device="cpu"):
    """q, k, v with entries in {-2, -1, 0, 1} (exact in fp16/bf16, and QK^T is
    exact in fp32 for d <= 128).  This is the CuTe DSL example's input trick
    for isolating softmax rounding from GEMM rounding."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = DTYPES[w.dtype]
    q = torch.randint(-2, 2, (w.B, w.Sq, w.Hq, w.d), generator=g).to(dt)
    k = torch.randint(-2, 2, (w.B, w.Sk, w.Hkv, w.d), generator=g).to(dt)
    v = torch.randint(-2, 2, (w.B, w.Sk, w.Hkv, w.d), generator=g).to(dt)
    if str(device) != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def make_paged_cache(k, v, lens, block_size: int, num_blocks: int | None = None,
                     seed: int = 0, fill: float = float("nan")):
    """Lay K and V out as a paged cache: pools of fixed-size blocks and a
    block table (the layout of attn_decode_paged).

    k, v: (B, S, Hkv, d) CPU tensors; sequence b keeps its first lens[b]
    rows.  Its j-th block of block_size tokens goes to a pool block whose id
    is drawn without replacement by ``randperm`` from a generator seeded
    with ``seed``, so the blocks of a sequence are scattered over the pool.
    Slots that hold no token are ``fill`` (NaN by default: a read of one
    shows in the result); table entries past a sequence's blocks are -1.
    num_blocks defaults to the blocks needed plus one per sequence.

    Returns (k_pool, v_pool, block_table, seqlens): pools (num_blocks,
    block_size, Hkv, d) of k's dtype, block_table int32 (B, max_blocks) with
    max_blocks the most blocks any sequence needs (at least 1), seqlens
    int32 (B,)."""
    B, S, Hkv, d = k.shape
    lens = [int(x) for x in lens]
    need = [max(0, -(-L // block_size)) for L in lens]
    total = sum(need)
    if num_blocks is None:
        num_blocks = total + B
    if num_blocks < max(total, 1):
        raise ValueError(f"{num_blocks} blocks cannot hold {total}")
    max_blocks = max(max(need), 1)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    ids = torch.randperm(num_blocks, generator=g)[:total].tolist()
    kp = torch.full((num_blocks, block_size, Hkv, d), fill, dtype=k.dtype)
    vp = torch.full((num_blocks, block_size, Hkv, d), fill, dtype=v.dtype)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    n = 0
    for b in range(B):
        for j in range(need[b]):
            lo, hi = j * block_size, min((j + 1) * block_size, lens[b])
            kp[ids[n], :hi - lo] = k[b, lo:hi]
            vp[ids[n], :hi - lo] = v[b, lo:hi]
            table[b, j] = ids[n]
            n += 1
    return kp, vp, table, torch.tensor(lens, dtype=torch.int32)
