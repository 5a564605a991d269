"""f32 grouped-query scaled dot-product attention for MI355X (gfx950).

The graph protocol's `attention` op, its KV-cache companion `cache_write`
and the `rope` op that precedes them (standalone, fused into cache_write and
fused into attention's q loads), and latent (MLA) attention in absorbed form,
as hand-written HIP kernels behind the C ABI in
include/attn.h (libattn.so). This package is the thin Python binding; it
has no fallback implementation and raises if the library is not built.
"""

from .attn import (AttnError, attn_cache_write, attn_cache_write2, attn_forward, attn_forward_append,
                   attn_forward_noalloc,
                   attn_last_error, attn_plan,
                   attn_rope, attn_rope_cache_write, attn_rope_table,
                   prepare_cache_write, prepare_cache_write2, prepare_forward, prepare_forward_append,
                   prepare_rope_cache_write,
                   attn_set_option, attn_timing_collect, attn_timing_enable, attn_validate,
                   attn_workspace_size, make_params, make_rope_params,
                   attn_mla_forward, attn_mla_plan, attn_mla_validate, attn_mla_workspace_size,
                   make_mla_params, prepare_mla_forward)
from ._lib import LIB_PATH, LibraryMissing

__all__ = [
    "AttnError", "LIB_PATH", "LibraryMissing", "attn_cache_write", "attn_cache_write2", "attn_forward",
    "attn_forward_append", "attn_last_error", "attn_plan", "attn_set_option", "attn_timing_collect",
    "attn_timing_enable", "attn_validate", "attn_workspace_size", "make_params",
    "prepare_cache_write", "prepare_cache_write2", "prepare_forward", "prepare_forward_append",
    "attn_rope", "attn_rope_cache_write", "attn_rope_table", "make_rope_params", "prepare_rope_cache_write",
    "attn_mla_forward", "attn_mla_plan", "attn_mla_validate", "attn_mla_workspace_size",
    "make_mla_params", "prepare_mla_forward", "attn_forward_noalloc",
]
