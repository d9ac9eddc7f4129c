"""Thin ctypes binding of ``libattn.so`` (the C ABI of ``include/attn.h``).

Argument marshalling only: every step of the attention forward runs in the HIP
kernels of the library.  torch is used for device memory and the current
stream.  There is no CPU fallback: if the library is missing, loading fails
with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIBRARY names another build of the same sources (the host-side
# sanitizer build used by the CPU checks)
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(PKG, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH = 0, 1, 2, 3
ATTN_ERR_SCRATCH = 4
ATTN_DTYPE_F16, ATTN_DTYPE_BF16, ATTN_DTYPE_F32 = 0, 1, 2
EXPORTED = ("attn_fwd", "attn_fwd_check", "attn_fwd_plan", "attn_fwd_split",
            "attn_fwd_split_noalloc",
            "attn_fwd_split_workspace", "attn_fwd_split_plan", "attn_fwd_strided",
            "attn_fwd_strided_check", "attn_merge", "attn_merge_check", "attn_bwd",
            "attn_bwd_check", "attn_bwd_workspace", "attn_bwd_causal_offset",
            "attn_bwd_causal_offset_check", "attn_fwd_causal_offset",
            "attn_fwd_causal_offset_check", "attn_fwd_causal_offset_workspace", "attn_decode_paged",
            "attn_decode_paged_check", "attn_decode_paged_workspace", "attn_status_str",
            "attn_abi_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_str(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime (soname libamdhip64.so.7, loaded by its
    # file name).  Loaded first, it satisfies libattn.so's dependency; loaded
    # after libattn.so, it maps a second runtime into the process beside
    # /opt/rocm's, and the two crash.  So torch goes first.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m exact_attention_19_amd.build`; "
            "there is no fallback implementation")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.restype = i
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_check.restype = i
    lib.attn_fwd_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i]
    lib.attn_fwd_plan.restype = i
    lib.attn_fwd_plan.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i), i]
    sz = ctypes.c_size_t
    lib.attn_fwd_split.restype = i
    lib.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.attn_fwd_split_noalloc.restype = i
    lib.attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
    lib.attn_fwd_split_workspace.restype = i
    lib.attn_fwd_split_workspace.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.attn_fwd_split_plan.restype = i
    lib.attn_fwd_split_plan.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(i), i]
    ll12 = ctypes.POINTER(ctypes.c_longlong)
    lib.attn_fwd_strided.restype = i
    lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, ll12, i,
                                     vp, sz, vp]
    lib.attn_fwd_strided_check.restype = i
    lib.attn_fwd_strided_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, ll12]
    lib.attn_bwd.restype = i
    lib.attn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_bwd_check.restype = i
    lib.attn_bwd_check.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i]
    lib.attn_bwd_workspace.restype = i
    lib.attn_bwd_workspace.argtypes = [i, i, i, ctypes.POINTER(sz)]
    lib.attn_merge.restype = i
    lib.attn_merge.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp, i, vp]
    lib.attn_merge_check.restype = i
    lib.attn_merge_check.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp, i]
    lo = ctypes.c_longlong
    lib.attn_fwd_causal_offset.restype = i
    lib.attn_fwd_causal_offset.argtypes = [vp] * 5 + [i] * 6 + [f, lo, i, vp, i, vp, sz, vp]
    lib.attn_fwd_causal_offset_check.restype = i
    lib.attn_fwd_causal_offset_check.argtypes = [vp] * 5 + [i] * 6 + [f, lo, i, vp]
    lib.attn_fwd_causal_offset_workspace.restype = i
    lib.attn_fwd_causal_offset_workspace.argtypes = [i] * 6 + [lo, i, i, ctypes.POINTER(sz)]
    lib.attn_bwd_causal_offset.restype = i
    lib.attn_bwd_causal_offset.argtypes = [vp] * 9 + [i] * 6 + [f, lo, i, vp, sz, vp]
    lib.attn_bwd_causal_offset_check.restype = i
    lib.attn_bwd_causal_offset_check.argtypes = [vp] * 9 + [i] * 6 + [f, lo, i]
    lib.attn_decode_paged.restype = i
    lib.attn_decode_paged.argtypes = [vp] * 7 + [i] * 9 + [f, i, i, i, vp, sz, vp]
    lib.attn_decode_paged_check.restype = i
    lib.attn_decode_paged_check.argtypes = [vp] * 7 + [i] * 9 + [f, i, i]
    lib.attn_decode_paged_workspace.restype = i
    lib.attn_decode_paged_workspace.argtypes = [i] * 7 + [ctypes.POINTER(sz)]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [i]
    lib.attn_abi_version.restype = i
    lib.attn_abi_version.argtypes = []
    _lib = lib
    return lib


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def attn_abi_version() -> int:
    return int(load_library().attn_abi_version())


def _dtype_code(t, allow_f32: bool = False) -> int:
    import torch
    if t.dtype == torch.float16:
        return ATTN_DTYPE_F16
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if allow_f32 and t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: q, k, v must be float16 or bfloat16")


def attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, causal, dtype_code) -> dict:
    """The launch attn_fwd would make (no device call)."""
    out = (ctypes.c_int * 11)()
    st = load_library().attn_fwd_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), dtype_code, out, 11)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_plan")
    keys = ("grid", "threads", "rows_per_wg", "keys_per_tile", "heads_per_wg",
            "rows_per_wave", "lds_bytes", "xcd_ordered", "pipelined", "decode", "key_halves")
    return dict(zip(keys, list(out)))


def attn_fwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Sq, Sk, Hq, Hkv, d,
                   scale, causal, dtype_code) -> int:
    """Validation only, on raw integer addresses; returns the status code."""
    return int(load_library().attn_fwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr,
                                             B, Sq, Sk, Hq, Hkv, d, float(scale),
                                             int(causal), dtype_code))


def attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, causal, dtype_code, kv_split=0) -> dict:
    """The launches attn_fwd_split would make (no device call)."""
    out = (ctypes.c_int * 7)()
    st = load_library().attn_fwd_split_plan(B, Sq, Sk, Hq, Hkv, d, int(causal), dtype_code,
                                            int(kv_split), out, 7)
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_split_plan")
    keys = ("grid", "pieces", "keys_per_piece", "first_split_row", "merge_grid", "threads",
            "key_halves")
    return dict(zip(keys, list(out)))


def attn_fwd_split_workspace(B, Sq, Sk, Hq, Hkv, d, causal, dtype_code, kv_split=0) -> int:
    """Workspace bytes attn_fwd_split needs (0 when it would not split)."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_fwd_split_workspace(B, Sq, Sk, Hq, Hkv, d, int(causal),
                                                 dtype_code, int(kv_split), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_split_workspace")
    return int(n.value)


def attn_merge_check(o_parts_ptr, lse_parts_ptr, n_parts, parts_dtype, B, Sq, Hq, d,
                     o_ptr, lse_ptr, dtype_code) -> int:
    """attn_merge's validation on raw integer addresses; returns the status."""
    return int(load_library().attn_merge_check(o_parts_ptr, lse_parts_ptr, n_parts,
                                               parts_dtype, B, Sq, Hq, d, o_ptr, lse_ptr,
                                               dtype_code))


def _check_qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (batch, seq, heads, d_head)")
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk = k.shape
    if tuple(v.shape) != (Bk, Sk, Hkv, dk) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _on_device(name, t, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (batch, seq, heads, d_head)")
    return B, Sq, Sk, Hq, Hkv, d, code


def _on_device(name, t, device):
    """A caller-given buffer the kernels write or read: a tensor on the GPU
    that holds q (a host tensor or one on another GPU would take a device
    address the kernel cannot use)."""
    if not hasattr(t, "is_cuda") or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")


def _check_lse(lse, B, Hq, Sq, device):
    import torch
    if lse is None:
        return
    _on_device("lse", lse, device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be a contiguous float32 (B, Hq, Sq) tensor")


def _check_workspace(workspace, device):
    if workspace is None:
        return
    _on_device("workspace", workspace, device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")


def _outputs(q, out, lse, return_lse):
    """out: (allocated here when None) a contiguous tensor with q's shape,
    dtype and device; lse: fp32 (B, Hq, Sq) on the same device, or None."""
    import torch
    B, Sq, Hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    _on_device("out", out, q.device)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {q.dtype} tensor of shape {tuple(q.shape)}")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Hq, Sq, q.device)
    return out, lse


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False,
             out=None, lse=None, return_lse: bool = True, stream=None):
    """O = softmax(scale * Q K^T + M) V and its LSE, on the GPU.

    q: (B, Sq, Hq, d); k, v: (B, Sk, Hkv, d); fp16 or bf16 CUDA tensors, dense.
    Returns (o, lse) with lse fp32 (B, Hq, Sq), or (o, None) if
    return_lse is False.  The launch goes to ``stream`` (a torch.cuda.Stream)
    or the current stream.
    """
    import torch
    B, Sq, Sk, Hq, Hkv, d, code = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse, return_lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)), code,
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return out, lse


def attn_fwd_split(q, k, v, scale: float | None = None, causal: bool = False,
                   kv_split: int = 0, out=None, lse=None, return_lse: bool = True,
                   workspace=None, stream=None):
    """attn_fwd with the keys of long query blocks split over workgroups and
    merged (for grids too small to fill the GPU).  kv_split: 0 = the
    library's choice, 1 = no split, k > 1 = at most k pieces per block.
    ``workspace`` is a uint8 CUDA tensor of at least attn_fwd_split_workspace
    bytes (allocated here when None).  Returns (o, lse) as attn_fwd does."""
    import torch
    B, Sq, Sk, Hq, Hkv, d, code = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse, return_lse)
    _check_workspace(workspace, q.device)
    if workspace is None:  # (a given workspace is size-checked by the library)
        need = attn_fwd_split_workspace(B, Sq, Sk, Hq, Hkv, d, causal, code, kv_split)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_fwd_split(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)), code, int(kv_split),
        ws_ptr, ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_split")
    return out, lse


def attn_fwd_split_noalloc(q, k, v, scale: float | None = None, causal: bool = False,
                           kv_split: int = 0, out=None, lse=None, stream=None):
    """attn_fwd_split with the key split's partial states in the library's
    static per-GPU scratch (no workspace, nothing allocated by the library).
    ``out`` and ``lse`` must be given (allocating them is the caller's
    business).  Calls whose kernels overlap on one GPU race on the scratch;
    calls on one stream are safe.  Raises AttnError (ATTN_ERR_SCRATCH) when
    the split needs more than the scratch holds."""
    import torch
    B, Sq, Sk, Hq, Hkv, d, code = _check_qkv(q, k, v)
    if out is None:
        raise ValueError("attn_fwd_split_noalloc writes into a caller-given out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse, False)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_fwd_split_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)), code, int(kv_split),
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_split_noalloc")
    return out, lse


def _strides_arg(vals):
    arr = (ctypes.c_longlong * 12)(*[int(x) for x in vals])
    return arr


def attn_fwd_strided_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Sq, Sk, Hq, Hkv, d,
                           scale, causal, dtype_code, strides) -> int:
    """attn_fwd_strided's validation on raw addresses and 12 element strides."""
    return int(load_library().attn_fwd_strided_check(
        q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Sq, Sk, Hq, Hkv, d, float(scale),
        int(causal), dtype_code, _strides_arg(strides)))


def attn_fwd_strided(q, k, v, scale: float | None = None, causal: bool = False,
                     layout: str = "bshd", kv_split: int = 0, out=None, lse=None,
                     return_lse: bool = True, workspace=None, stream=None):
    """attn_fwd on strided views: q, k, v (and ``out``) may be any views whose
    last dimension is contiguous, e.g. slices of a packed QKV projection.

    layout "bshd": q is (B, Sq, Hq, d) and k, v are (B, Sk, Hkv, d);
    layout "bhsd": q is (B, Hq, Sq, d) and k, v are (B, Hkv, Sk, d).
    ``out`` (allocated here, dense, when None) has the layout of q.  lse is
    (B, Hq, Sq) fp32.  kv_split and workspace as for attn_fwd_split."""
    import torch
    if layout not in ("bshd", "bhsd"):
        raise ValueError("layout must be 'bshd' or 'bhsd'")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    # logical (b, s, h, c) views
    view = (lambda t: t) if layout == "bshd" else (lambda t: t.transpose(1, 2))
    qv, kv_, vv, ov = view(q), view(k), view(v), view(out)
    B, Sq, Hq, d = qv.shape
    Bk, Sk, Hkv, dk = kv_.shape
    if tuple(vv.shape) != (Bk, Sk, Hkv, dk) or Bk != B or dk != d or tuple(ov.shape) != (B, Sq, Hq, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, out {tuple(out.shape)} ({layout})")
    code = _dtype_code(q)
    for name, t in (("q", qv), ("k", kv_), ("v", vv), ("out", ov)):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v and out must share one dtype")
        _on_device(name, t, q.device)
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Hq, Sq, q.device)
    _check_workspace(workspace, q.device)
    strides = []
    for t in (qv, kv_, vv, ov):
        strides += [t.stride(0), t.stride(1), t.stride(2)]
    if workspace is None:
        need = attn_fwd_split_workspace(B, Sq, Sk, Hq, Hkv, d, causal, code, kv_split)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_fwd_strided(
        qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), ov.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)), code, _strides_arg(strides),
        int(kv_split), ws_ptr, ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_strided")
    return out, lse


def attn_fwd_causal_offset_workspace(B, Sq, Sk, Hq, Hkv, d, causal_offset, dtype_code,
                                     kv_split=0) -> int:
    """Workspace bytes attn_fwd_causal_offset needs (0 when it does not split)."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_fwd_causal_offset_workspace(B, Sq, Sk, Hq, Hkv, d, int(causal_offset),
                                                         dtype_code, int(kv_split),
                                                         ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_causal_offset_workspace")
    return int(n.value)


def attn_fwd_causal_offset(q, k, v, causal_offset: int, scale: float | None = None,
                           kv_split: int = 0, out=None, lse=None, return_lse: bool = True,
                           workspace=None, stream=None):
    """Causal attention with an explicit mask offset: query i sees key j iff
    j <= i + causal_offset.  For keys [k0, k1) of a causal problem with Sk
    keys in all, causal_offset = Sk - Sq - k0 (k, v may then be the slices
    k[:, k0:k1], v[:, k0:k1] of the full tensors: any (b, s, h) strides with
    a contiguous last dimension).  q, k, v in the (B, S, H, d) layout; out
    dense unless given.  Returns (o, lse); rows that see no key get o = 0,
    lse = -inf.  The shards' (o, lse) merge with attn_merge."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (batch, seq, heads, d_head)")
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk = k.shape
    if tuple(v.shape) != (Bk, Sk, Hkv, dk) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}")
    code = _dtype_code(q)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v and out must share one dtype")
        _on_device(name, t, q.device)
        if t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    if tuple(out.shape) != (B, Sq, Hq, d):
        raise ValueError("out must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, Hq, Sq, q.device)
    _check_workspace(workspace, q.device)
    strides = []
    for t in (q, k, v, out):
        strides += [t.stride(0), t.stride(1), t.stride(2)]
    if workspace is None:
        need = attn_fwd_causal_offset_workspace(B, Sq, Sk, Hq, Hkv, d, causal_offset, code,
                                                kv_split)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_fwd_causal_offset(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, B, Sq, Sk, Hq, Hkv, d, float(scale),
        int(causal_offset), code, _strides_arg(strides), int(kv_split), ws_ptr, ws_bytes,
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_causal_offset")
    return out, lse


def attn_merge(o_parts, lse_parts, dtype=None, out=None, lse=None,
               return_lse: bool = True, stream=None):
    """Merge partial attention states over disjoint key subsets.

    o_parts: (P, B, Sq, Hq, d) CUDA tensor, float32, float16 or bfloat16, each
    part normalised over its own keys; lse_parts: (P, B, Hq, Sq) float32
    (-inf = the part saw no key).  dtype: the output dtype (torch.float16 or
    torch.bfloat16; default: that of o_parts, or bfloat16 for float32 parts).
    Returns (o, lse) of the union: o (B, Sq, Hq, d), lse (B, Hq, Sq)."""
    import torch
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be (P, B, Sq, Hq, d) and lse_parts (P, B, Hq, Sq)")
    P, B, Sq, Hq, d = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, Hq, Sq) or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be a float32 (P, B, Hq, Sq) tensor")
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        _on_device(name, t, o_parts.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    pcode = _dtype_code(o_parts, allow_f32=True)
    if dtype is None:
        dtype = torch.bfloat16 if o_parts.dtype == torch.float32 else o_parts.dtype
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=dtype, device=o_parts.device)
    _on_device("out", out, o_parts.device)
    ocode = _dtype_code(out)
    if tuple(out.shape) != (B, Sq, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, Sq, Hq, d) tensor")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=o_parts.device)
    _check_lse(lse, B, Hq, Sq, o_parts.device)
    if stream is None:
        stream = torch.cuda.current_stream(o_parts.device)
    st = load_library().attn_merge(
        o_parts.data_ptr(), lse_parts.data_ptr(), P, pcode, B, Sq, Hq, d, out.data_ptr(),
        lse.data_ptr() if lse is not None else None, ocode,
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_merge")
    return out, lse


def attn_bwd_workspace(B, Sq, Hq) -> int:
    """Workspace bytes attn_bwd needs (two fp32 values per query row)."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_bwd_workspace(B, Sq, Hq, ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_workspace")
    return int(n.value)


def attn_bwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr,
                   B, Sq, Sk, Hq, Hkv, d, scale, causal, dtype_code) -> int:
    """attn_bwd's validation on raw addresses; returns the status code."""
    return int(load_library().attn_bwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr,
                                             dq_ptr, dk_ptr, dv_ptr, B, Sq, Sk, Hq, Hkv, d,
                                             float(scale), int(causal), dtype_code))


def attn_bwd_causal_offset_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                 dv_ptr, B, Sq, Sk, Hq, Hkv, d, scale, causal_offset,
                                 dtype_code) -> int:
    """attn_bwd_causal_offset's validation on raw addresses; returns the status code."""
    return int(load_library().attn_bwd_causal_offset_check(
        q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, B, Sq, Sk, Hq, Hkv,
        d, float(scale), ctypes.c_longlong(int(causal_offset)), dtype_code))


def _bwd_args(q, k, v, o, lse, dout, scale, dq, dk, dv, workspace, stream):
    import torch
    B, Sq, Sk, Hq, Hkv, d, code = _check_qkv(q, k, v)
    for name, t in (("o", o), ("dout", dout)):
        _on_device(name, t, q.device)
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor like q")
    if lse is None:
        raise ValueError("lse (the forward's, fp32 (B, Hq, Sq)) is required")
    _check_lse(lse, B, Hq, Sq, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _on_device(name, t, q.device)
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor shaped like its input")
    _check_workspace(workspace, q.device)
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace(B, Sq, Hq), dtype=torch.uint8,
                                device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            B, Sq, Sk, Hq, Hkv, d, float(scale))
    tail = (code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream.cuda_stream))
    return head, tail, (dq, dk, dv)


def attn_bwd(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * o) for o, lse = attn_fwd(q, k, v).

    q, o, dout: (B, Sq, Hq, d); k, v: (B, Sk, Hkv, d); one dtype (fp16/bf16),
    dense; lse: (B, Hq, Sq) fp32 from attn_fwd.  Outputs are allocated when
    not given; ``workspace`` (uint8, attn_bwd_workspace bytes) likewise."""
    head, tail, out = _bwd_args(q, k, v, o, lse, dout, scale, dq, dk, dv, workspace, stream)
    st = load_library().attn_bwd(*head, int(bool(causal)), *tail)
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return out


def attn_bwd_causal_offset(q, k, v, o, lse, dout, causal_offset: int,
                           scale: float | None = None, dq=None, dk=None, dv=None,
                           workspace=None, stream=None):
    """Backward of one causal key shard: query i sees key j of k/v iff
    j <= i + causal_offset.  o and lse are the FULL problem's (the merged
    forward over all shards); the returned dk, dv are this shard's exact
    gradients and dq is its part of the full dQ (the parts of all shards sum
    to it).  Arguments otherwise as for attn_bwd."""
    head, tail, out = _bwd_args(q, k, v, o, lse, dout, scale, dq, dk, dv, workspace, stream)
    st = load_library().attn_bwd_causal_offset(*head, ctypes.c_longlong(int(causal_offset)),
                                               *tail)
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_causal_offset")
    return out

def attn_decode_paged_check(q_ptr, k_ptr, v_ptr, table_ptr, lens_ptr, o_ptr, lse_ptr, B, Sq,
                            Hq, Hkv, d, num_blocks, block_size, max_blocks, max_seqlen, scale,
                            causal, dtype_code) -> int:
    """attn_decode_paged's validation on raw integer addresses; returns the status."""
    return int(load_library().attn_decode_paged_check(
        q_ptr, k_ptr, v_ptr, table_ptr, lens_ptr, o_ptr, lse_ptr, B, Sq, Hq, Hkv, d,
        num_blocks, block_size, max_blocks, max_seqlen, float(scale), int(causal), dtype_code))


def attn_decode_paged_workspace(B, Sq, Hq, Hkv, d, max_seqlen, kv_split=0) -> int:
    """Workspace bytes attn_decode_paged needs (0 when it does not split)."""
    n = ctypes.c_size_t(0)
    st = load_library().attn_decode_paged_workspace(B, Sq, Hq, Hkv, d, max_seqlen,
                                                    int(kv_split), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged_workspace")
    return int(n.value)


def attn_decode_paged(q, k_cache, v_cache, block_table, seqlens, scale: float | None = None,
                      causal: bool = True, max_seqlen: int | None = None, kv_split: int = 0,
                      out=None, lse=None, return_lse: bool = True, workspace=None,
                      stream=None):
    """Decode attention over a paged K/V cache.

    q: (B, Sq, Hq, d); k_cache, v_cache: (num_blocks, block_size, Hkv, d);
    block_table: int32 (B, max_blocks); seqlens: int32 (B,), all on the GPU.
    Sequence b attends to its first seqlens[b] tokens, token t at
    block_table[b, t // block_size], slot t % block_size; its Sq queries are
    its last Sq positions.  ``max_seqlen`` (default: the table's capacity,
    max_blocks * block_size) bounds the lengths and sizes the key split;
    it is never read from the device.  Returns (o, lse) as attn_fwd does."""
    import torch
    if q.dim() != 4 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be (B, Sq, Hq, d) and k_cache, v_cache one "
                         "(num_blocks, block_size, Hkv, d) shape")
    B, Sq, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError(f"head size mismatch: q {d}, cache {dk}")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if block_table.dtype != torch.int32 or seqlens.dtype != torch.int32:
        raise TypeError("block_table and seqlens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seqlens.shape) != (B,):
        raise ValueError("block_table must be (B, max_blocks) and seqlens (B,)")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seqlens", seqlens)):
        _on_device(name, t, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    max_blocks = block_table.shape[1]
    if max_seqlen is None:
        max_seqlen = max_blocks * block_size
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse, return_lse)
    _check_workspace(workspace, q.device)
    if workspace is None:
        need = attn_decode_paged_workspace(B, Sq, Hq, Hkv, d, int(max_seqlen), kv_split)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = load_library().attn_decode_paged(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        seqlens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, Sq, Hq, Hkv, d, num_blocks, block_size, max_blocks, int(max_seqlen), float(scale),
        int(bool(causal)), code, int(kv_split), ws_ptr, ws_bytes,
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged")
    return out, lse
