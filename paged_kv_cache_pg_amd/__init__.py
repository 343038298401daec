"""Paged KV-cache attention for AMD MI355X (gfx950)."""
