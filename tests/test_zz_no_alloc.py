"""attn_fwd_split_noalloc (the library's static scratch instead of a caller
workspace) against attn_fwd_split through the C ABI, and both against the
fp64 oracle: two calls in a row on one stream, the second smaller, so the
second reuses the scratch the first left behind."""
import ctypes
import math

import numpy as np
import pytest
import torch

from exact_attention_19_amd.workloads import WORKLOADS, Workload, make_inputs
from parity_common import _check_full, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_19_amd import load_library
    load_library()  # fail loudly if the HIP library is missing


def _call_noalloc(lib, q, k, v, o, lse, w, code, kv_split, stream):
    return lib.attn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d,
                                      ctypes.c_float(w.scale), int(w.causal), code, kv_split,
                                      ctypes.c_void_p(stream.cuda_stream))


def test_noalloc_matches_workspace_path_two_calls():
    from exact_attention_19_amd import attn_fwd_split, attn_fwd_split_workspace, load_library
    from exact_attention_19_amd.binding import ATTN_DTYPE_BF16, ATTN_DTYPE_F16, ATTN_OK
    lib = load_library()
    stream = torch.cuda.current_stream()
    big = WORKLOADS["mha_causal_offset_f16_b1_h16_sq1280_sk1536_d128"]
    small = Workload("noalloc_small", 2, 8, 2, 300, 1000, 128, "bf16", True, 1 / math.sqrt(128))
    runs = [(big, 2), (small, 4)]  # both split: pieces in the scratch
    outs = []
    for w, kv_split in runs:
        code = ATTN_DTYPE_BF16 if w.dtype == "bf16" else ATTN_DTYPE_F16
        need = attn_fwd_split_workspace(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d, w.causal, code,
                                        kv_split)
        assert 0 < need <= lib_scratch_bytes(), (w.name, need)
        q, k, v = make_inputs(w, seed=11)
        qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
        o = torch.full_like(qg, float("nan"))
        lse = torch.full((w.B, w.Hq, w.Sq), float("nan"), dtype=torch.float32, device="cuda")
        _say(f"[gpu] attn_fwd_split_noalloc {w.name} kv_split={kv_split} (needs {need} bytes)")
        assert _call_noalloc(lib, qg, kg, vg, o, lse, w, code, kv_split, stream) == ATTN_OK
        outs.append((w, kv_split, q, k, v, qg, kg, vg, o, lse))
    torch.cuda.synchronize()
    for w, kv_split, q, k, v, qg, kg, vg, o, lse in outs:
        o_ws, lse_ws = attn_fwd_split(qg, kg, vg, scale=w.scale, causal=w.causal,
                                      kv_split=kv_split)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical bits
        assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws), w.name
        _check_full(w, q, k, v, o.cpu(), lse.cpu(), strict=False)


def test_noalloc_without_split_and_too_large():
    from exact_attention_19_amd import attn_fwd, attn_fwd_split_noalloc
    from exact_attention_19_amd.binding import ATTN_ERR_SCRATCH, AttnError
    w = Workload("noalloc_nosplit", 1, 8, 2, 200, 333, 64, "f16", True, 0.125)
    q, k, v = (t.cuda() for t in make_inputs(w, seed=2))
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, 200), dtype=torch.float32, device="cuda")
    attn_fwd_split_noalloc(q, k, v, scale=w.scale, causal=True, kv_split=1, out=o, lse=lse)
    o2, l2 = attn_fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    # a split whose partial states exceed the scratch is refused, nothing launched
    wl = Workload("noalloc_big", 4, 32, 8, 8192, 8192, 128, "bf16", True, 0.1)
    ql = torch.empty((wl.B, wl.Sq, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda")
    kl = torch.empty((wl.B, wl.Sk, wl.Hkv, wl.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnError) as e:
        attn_fwd_split_noalloc(ql, kl, kl, scale=wl.scale, causal=True, kv_split=8,
                               out=torch.empty_like(ql))
    assert e.value.status == ATTN_ERR_SCRATCH


def lib_scratch_bytes():
    import re
    import os
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "include", "attn.h")
    m = re.search(r"#define\s+ATTN_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)",
                  open(hdr).read())
    return int(m.group(1)) << int(m.group(2))
