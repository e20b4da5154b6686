"""Causal grouped-query attention with RoPE for AMD MI355X (gfx950)."""
