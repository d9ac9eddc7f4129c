"""ctypes front end of the fp64 C oracle (test infrastructure only).

The attention arithmetic lives in ``attn_oracle.c``; this module widens
inputs to fp64, passes pointers and reshapes the outputs.  The merge of
partial states (``merge_partials_oracle``) is written here in numpy fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
# ATTN_ORACLE_LIBRARY names another build of the same source (the sanitizer
# build below) for the test run that checks it.
_LIB = os.environ.get("ATTN_ORACLE_LIBRARY") or os.path.join(_HERE, "libattn_oracle.so")
_SANITIZE_LIB = os.path.join(os.path.dirname(_HERE), "_build", "sanitize", "libattn_oracle.so")
_lib = None


def oracle_lib_path() -> str:
    return _LIB


def build_oracle(force: bool = True, sanitize: bool = False) -> str:
    """Compile attn_oracle.c into libattn_oracle.so with gcc (-O2, no fast-math:
    the oracle keeps IEEE fp64 semantics).  sanitize=True: a separate build
    with AddressSanitizer and UndefinedBehaviorSanitizer, compiled by the
    ROCm clang so that it shares one sanitizer runtime with the HIP library's
    host-side sanitizer build in the process that tests both."""
    lib = _SANITIZE_LIB if sanitize else _LIB
    if force or not os.path.exists(lib):
        os.makedirs(os.path.dirname(lib), exist_ok=True)
        tmp = lib + ".tmp"
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c99", "-fPIC", "-shared",
                   "-pthread", "-ffp-contract=off", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
        else:
            cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                   "-fno-fast-math", "-ffp-contract=off"]
        subprocess.check_call(cmd + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_attn_fwd_range
        f.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        f.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                      ctypes.c_double, ctypes.c_int, i64, i64,
                      ctypes.POINTER(ctypes.c_int64), i64, ctypes.c_int]
        g = lib.oracle_attn_bwd
        g.restype = ctypes.c_int
        g.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                      ctypes.c_double, ctypes.c_int, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16
    (a machine shared by several GPUs' jobs may give each a 16-CPU share
    whatever the affinity mask reports)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _as_f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (any float dtype) to a
    contiguous fp64 numpy array.  Widening fp16/bf16/fp32 to fp64 is exact."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attn_fwd_oracle(q, k, v, scale: float, causal: bool, rows=None,
                    nthreads: int | None = None, key_range=None):
    """Exact attention forward in fp64.

    q: (B, Sq, Hq, d); k, v: (B, Sk, Hkv, d).  Returns (o, lse):
      rows is None -> o (B, Sq, Hq, d), lse (B, Hq, Sq)
      rows given   -> rows are flat ids (b*Hq + h)*Sq + i; o (n, d), lse (n,)
    key_range=(k0, k1) keeps only keys k0 <= j < k1 (the causal rule still
    counts j against the full key length): the partial state of each row over
    that key subset, o normalised over those keys and lse their log-sum-exp
    (o = 0, lse = -inf where no key of the range is visible).
    """
    qd, kd, vd = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Sq, Hq, d = qd.shape
    Bk, Sk, Hkv, dk = kd.shape
    if vd.shape != kd.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k, v")
    if nthreads is None:
        nthreads = default_threads()
    dp = ctypes.POINTER(ctypes.c_double)
    if rows is None:
        o = np.empty((B, Sq, Hq, d), np.float64)
        lse = np.empty((B, Hq, Sq), np.float64)
        rows_p, n = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = int(r.size)
        o = np.empty((n, d), np.float64)
        lse = np.empty((n,), np.float64)
        rows_p = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    k0, k1 = (0, Sk) if key_range is None else (int(key_range[0]), int(key_range[1]))
    rc = _load().oracle_attn_fwd_range(
        qd.ctypes.data_as(dp), kd.ctypes.data_as(dp), vd.ctypes.data_as(dp),
        o.ctypes.data_as(dp), lse.ctypes.data_as(dp),
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)), k0, k1,
        rows_p, n, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd failed with code {rc}")
    return o, lse


def gather_paged_oracle(cache, block_table, b: int, length: int) -> np.ndarray:
    """The first ``length`` tokens of sequence b from a paged pool, in order.

    cache: (num_blocks, block_size, Hkv, d); block_table: (B, max_blocks)
    integers.  Token t of sequence b sits in block block_table[b, t //
    block_size] at slot t % block_size: a paged K/V cache is an address
    translation in front of a dense per-sequence key array (the MiniPaged-
    Qwen page, section 19, names Paged Attention for decode and gives no
    layout; this is the plainest one).  cache may be a numpy array or a CPU
    torch tensor of any float dtype.  Returns (length, Hkv, d) fp64."""
    bt = np.asarray(block_table, dtype=np.int64)
    bs = cache.shape[1]
    t = np.arange(length)
    blocks, slots = bt[b, t // bs], t % bs  # where token t lives
    if hasattr(cache, "detach"):  # torch tensor: index it before widening
        import torch
        rows = cache.detach()[torch.from_numpy(blocks), torch.from_numpy(slots)]
    else:
        rows = np.asarray(cache)[blocks, slots]
    return _as_f64(rows)


def attn_decode_paged_oracle(q, k_cache, v_cache, block_table, seqlens, scale: float,
                             causal: bool, max_seqlen: int | None = None):
    """Attention of each sequence's Sq query tokens over its paged K/V history.

    q: (B, Sq, Hq, d); k_cache, v_cache: (num_blocks, block_size, Hkv, d);
    block_table: (B, max_blocks); seqlens: (B,).  Sequence b has L_b =
    min(seqlens[b], max_seqlen) keys (max_seqlen defaults to no bound; a
    length <= 0 means none), gathered by ``gather_paged_oracle``; its queries
    are its last Sq positions, so the causal mask is bottom-right aligned to
    L_b.  Each sequence is then exactly the dense forward: attn_fwd_oracle
    with Sk = L_b.  Returns o (B, Sq, Hq, d), lse (B, Hq, Sq); rows that see
    no key get o = 0, lse = -inf."""
    qd = _as_f64(q)
    B, Sq, Hq, d = qd.shape
    lens = np.asarray(seqlens, dtype=np.int64).reshape(-1)
    o = np.zeros((B, Sq, Hq, d), np.float64)
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        L = int(lens[b]) if max_seqlen is None else min(int(lens[b]), int(max_seqlen))
        if L <= 0:
            continue
        kb = gather_paged_oracle(k_cache, block_table, b, L)[None]
        vb = gather_paged_oracle(v_cache, block_table, b, L)[None]
        ob, lb = attn_fwd_oracle(qd[b:b + 1], kb, vb, scale, causal)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def merge_partials_oracle(o_parts, lse_parts):
    """Combine partial attention states over disjoint key subsets, in fp64.

    o_parts: (P, B, Sq, Hq, d) outputs, each normalised over its own keys;
    lse_parts: (P, B, Hq, Sq) natural-log sums of exp of the scaled scores of
    those keys (-inf for a row that saw no key).  Returns (o, lse) of the
    union of the key subsets, o (B, Sq, Hq, d) and lse (B, Hq, Sq).

    This is the online-softmax state update ("FlashAttention personal
    implementation notes", section "Online Softmax": m_new = max(m_old, m_t),
    alpha = e^(m_old - m_new), l_new = alpha l_old + (tile sum),
    O~_new = alpha O~_old + (tile numerator)), applied with whole parts in the
    place of tiles.  A normalised part (O_p, lse_p) is the state m = lse_p,
    l = 1, O~ = O_p: it has the same ratio O~/l and the same m + ln l, so
    each part enters with a tile weight e^(lse_p - m_new).  The result is
    O = O~ / l and lse = m + ln l; a row that no part saw stays o = 0,
    lse = -inf.
    """
    op = np.asarray(o_parts, dtype=np.float64)
    lp = np.asarray(lse_parts, dtype=np.float64)
    P, B, Sq, Hq, d = op.shape
    if lp.shape != (P, B, Hq, Sq):
        raise ValueError(f"lse_parts must be {(P, B, Hq, Sq)}, got {lp.shape}")
    # move to (P, B, Hq, Sq, d) so that a part's row state lines up with its lse
    op = op.transpose(0, 1, 3, 2, 4)
    m = np.full((B, Hq, Sq), -np.inf)
    l = np.zeros((B, Hq, Sq))
    acc = np.zeros((B, Hq, Sq, d))
    for t in range(P):
        m_t = lp[t]
        m_new = np.maximum(m, m_t)
        seen = np.isfinite(m_new)
        # e^(m_old - m_new) and e^(m_t - m_new); rows no part has seen yet
        # keep alpha = beta = 0 and their zero state
        with np.errstate(invalid="ignore"):
            alpha = np.where(seen, np.exp(m - np.where(seen, m_new, 0.0)), 0.0)
            beta = np.where(seen, np.exp(m_t - np.where(seen, m_new, 0.0)), 0.0)
        l = alpha * l + beta * 1.0
        acc = alpha[..., None] * acc + beta[..., None] * op[t]
        m = m_new
    seen = l > 0
    o = np.where(seen[..., None], acc / np.where(seen, l, 1.0)[..., None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return o.transpose(0, 2, 1, 3).copy(), lse


def attn_bwd_oracle(q, k, v, dout, scale: float, causal: bool, nthreads: int | None = None):
    """Gradients (dq, dk, dv) of sum(dout * O) in fp64, O the attention
    forward of (q, k, v); shapes as for attn_fwd_oracle, dout like q.  The
    arithmetic is attn_oracle.c's oracle_attn_bwd (chain rule through the
    two-pass softmax definition)."""
    qd, kd, vd, dod = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    B, Sq, Hq, d = qd.shape
    Bk, Sk, Hkv, dk_ = kd.shape
    if vd.shape != kd.shape or Bk != B or dk_ != d or dod.shape != qd.shape:
        raise ValueError("shape mismatch between q, k, v, dout")
    if nthreads is None:
        nthreads = default_threads()
    dq = np.empty_like(qd)
    dk = np.empty_like(kd)
    dv = np.empty_like(vd)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attn_bwd(
        qd.ctypes.data_as(dp), kd.ctypes.data_as(dp), vd.ctypes.data_as(dp),
        dod.ctypes.data_as(dp), dq.ctypes.data_as(dp), dk.ctypes.data_as(dp),
        dv.ctypes.data_as(dp), B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)),
        int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed with code {rc}")
    return dq, dk, dv
