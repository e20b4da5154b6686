"""Causal grouped-query attention with RoPE for AMD MI355X (gfx950).

The compute lives in libne_rope_attn.so (hand-written HIP kernels behind the C ABI of
include/ne_rope_attn.h); `binding` marshals torch tensors to it, and raises if it is missing.
"""
from .binding import (NeError, bwd_workspace_bytes, decode_workspace_bytes, fwd_workspace_bytes,  # noqa: F401
                      kv_cache_bytes, lib, ne_kv_cache_append, ne_rope_attn_bwd, ne_rope_attn_bwd_window,
                      ne_rope_attn_bwd_ex, ne_rope_attn_decode, ne_rope_attn_fwd, ne_rope_attn_fwd_ex,
                      ne_rope_attn_fwd_window, ne_qkv_rope_proj, new_kv_cache)
