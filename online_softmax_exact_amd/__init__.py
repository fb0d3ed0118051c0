"""Exact blocked attention for AMD Instinct MI355X (gfx950).

The computation runs in the HIP library ``libattn_mi355x.so`` (C ABI declared
in ``include/attn_mi355x.h``); this package is its Python binding.  The
library is loaded on first use and a missing library raises at once.
"""
from ._lib import (attn_bwd, attn_decode_splitkv, attn_decode_splitkv_noalloc,
                   attn_decode_workspace_bytes, attn_fwd, attn_merge_states, load_library,
                   split_workspace_views, strerror)

__all__ = ["attn_fwd", "attn_bwd", "attn_decode_splitkv", "attn_decode_splitkv_noalloc",
           "attn_decode_workspace_bytes", "attn_merge_states", "load_library",
           "split_workspace_views", "strerror"]
