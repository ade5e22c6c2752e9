"""Paged KV-cache attention for AMD Instinct MI355X (gfx950)."""
