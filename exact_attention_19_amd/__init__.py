"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

``attn_fwd`` runs the HIP kernel of ``libattn.so`` through its C ABI
(``include/attn.h``); ``attn_fwd_split`` splits the keys of long query blocks
over workgroups and merges them (small grids), and ``attn_fwd_split_noalloc``
does the same in the library's static scratch; ``attn_fwd_strided`` takes
strided views (e.g. the (B, H, S, d) layout); ``attn_merge`` combines
partial states over disjoint key subsets; ``attn_bwd`` gives dQ, dK, dV;
``attn_decode_paged`` runs decode attention over a paged K/V cache;
``attn_fwd_causal_offset`` and ``attn_bwd_causal_offset`` take the causal
mask's offset explicitly (a key shard of a longer causal problem).  The
library is loaded on first use; if it has not been built, that call raises
ImportError (there is no fallback path).
"""
from .binding import (  # noqa: F401
    AttnError, attn_abi_version, attn_bwd, attn_bwd_causal_offset,
    attn_bwd_causal_offset_check, attn_bwd_check, attn_bwd_workspace,
    attn_decode_paged, attn_decode_paged_check, attn_decode_paged_workspace, attn_fwd,
    attn_fwd_causal_offset, attn_fwd_causal_offset_workspace,
    attn_fwd_check, attn_fwd_plan, attn_fwd_split, attn_fwd_split_noalloc, attn_fwd_split_plan,
    attn_fwd_split_workspace, attn_fwd_strided, attn_fwd_strided_check, attn_merge,
    attn_merge_check, attn_status_str, load_library)
