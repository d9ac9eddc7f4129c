"""The C ABI without a GPU: the library loads, exports every symbol that
include/attn.h declares, and rejects bad arguments before any device call."""
import ctypes
import math
import os
import re

import pytest

from exact_attention_19_amd import binding
from exact_attention_19_amd.binding import (ATTN_DTYPE_BF16, ATTN_DTYPE_F16,
                                            ATTN_ERR_INVALID_ARG,
                                            ATTN_ERR_UNSUPPORTED, ATTN_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_19_amd.build import build_library
        build_library()
    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define\s+ATTN_ABI_VERSION\s+(\d+)", open(HEADER).read())
    _lib()
    assert binding.attn_abi_version() == int(m.group(1))


def test_status_strings():
    _lib()
    assert binding.attn_status_str(ATTN_OK) == "ok"
    assert "invalid" in binding.attn_status_str(ATTN_ERR_INVALID_ARG)
    assert "unsupported" in binding.attn_status_str(ATTN_ERR_UNSUPPORTED)
    assert binding.attn_status_str(99) == "unknown status"


# fake, 16-byte aligned addresses: validation never dereferences them
A = 0x10000
GOOD = dict(q=A, k=A + 0x1000, v=A + 0x2000, o=A + 0x3000, lse=A + 0x4000,
            B=2, Sq=100, Sk=120, Hq=8, Hkv=2, d=128, scale=0.125, causal=1,
            dtype=ATTN_DTYPE_BF16)


def _check(**over):
    a = dict(GOOD, **over)
    return binding.attn_fwd_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                  a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["d"],
                                  a["scale"], a["causal"], a["dtype"])


def test_valid_arguments_pass_validation():
    _lib()
    assert _check() == ATTN_OK
    assert _check(lse=None) == ATTN_OK
    assert _check(d=64, dtype=ATTN_DTYPE_F16, causal=0) == ATTN_OK
    # the largest head count whose 64-row tile stays below 2^31 bytes
    assert _check(Hq=(1 << 17) - 8, Hkv=(1 << 17) - 8, B=1, Sq=1, Sk=1) == ATTN_OK


@pytest.mark.parametrize("over", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(B=0), dict(Sq=0), dict(Sk=0), dict(Hq=0), dict(Hkv=0), dict(d=0),
    dict(Sq=-3), dict(Hq=6, Hkv=4),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")),
    dict(scale=float("inf")), dict(causal=2), dict(causal=-1),
    dict(q=A + 8), dict(o=A + 0x3002), dict(lse=A + 0x4002),
    dict(Sq=1 << 29, Sk=1 << 29),
    # a 64-row K/V tile must span less than 2^31 bytes: Hkv * d * 2 * 64
    dict(Hq=1 << 17, Hkv=1 << 17, B=1, Sq=1, Sk=1),
])
def test_invalid_arguments(over):
    _lib()
    assert _check(**over) == ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("over", [dict(d=96), dict(d=256), dict(d=32),
                                  dict(dtype=2), dict(dtype=-1)])
def test_unsupported(over):
    _lib()
    assert _check(**over) == ATTN_ERR_UNSUPPORTED


def test_attn_fwd_rejects_before_any_device_call():
    """attn_fwd with bad arguments returns the validation status without
    touching HIP (safe here, where there is no GPU)."""
    lib = _lib()
    st = lib.attn_fwd(A, A, A, A, None, 1, 8, 8, 4, 3, 64, ctypes.c_float(1.0), 0,
                      ATTN_DTYPE_F16, None)
    assert st == ATTN_ERR_INVALID_ARG
    st = lib.attn_fwd(A, A, A, A, None, 1, 8, 8, 4, 4, 80, ctypes.c_float(1.0), 0,
                      ATTN_DTYPE_F16, None)
    assert st == ATTN_ERR_UNSUPPORTED


def test_plan_matches_the_kernel_geometry():
    _lib()
    # GQA group of 4: four heads share each workgroup's K/V tiles
    p = binding.attn_fwd_plan(1, 8192, 8192, 32, 8, 128, 1, ATTN_DTYPE_BF16)
    assert p["heads_per_wg"] == 4
    assert p["threads"] % 64 == 0
    assert p["grid"] == math.ceil(8192 / p["rows_per_wg"]) * 8 * (4 // p["heads_per_wg"])
    assert p["xcd_ordered"] == 1
    assert p["lds_bytes"] <= 160 * 1024
    # MHA: heads are not packed; row blocks are
    p = binding.attn_fwd_plan(2, 1024, 1024, 16, 16, 128, 1, ATTN_DTYPE_F16)
    assert p["heads_per_wg"] == 1
    assert p["grid"] == math.ceil(1024 / p["rows_per_wg"]) * 2 * 16
    # tiny: fewer than 8 columns, no XCD grouping
    p = binding.attn_fwd_plan(1, 128, 128, 2, 2, 64, 0, ATTN_DTYPE_F16)
    assert p["xcd_ordered"] == 0


def test_plan_rejects_bad_sizes():
    _lib()
    with pytest.raises(binding.AttnError):
        binding.attn_fwd_plan(1, 0, 8, 4, 4, 64, 0, ATTN_DTYPE_F16)
