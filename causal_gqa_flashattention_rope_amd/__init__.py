"""Causal grouped-query attention with RoPE for AMD MI355X (gfx950).

The compute lives in libne_rope_attn.so (hand-written HIP kernels behind the C ABI of
include/ne_rope_attn.h); `binding` marshals torch tensors to it, and raises if it is missing.
"""
from .binding import (NeError, decode_workspace_bytes, kv_cache_bytes, lib, ne_kv_cache_append,  # noqa: F401
                      ne_qkv_rope_proj, ne_rope_attn_bwd, ne_rope_attn_bwd_ex, ne_rope_attn_decode, ne_rope_attn_fwd,
                      ne_rope_attn_fwd_ex, ne_rope_table_check, ne_rope_table_init, new_kv_cache, new_workspace,
                      workspace_bytes)
