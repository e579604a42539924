"""Paged-KV decode attention and K/V append for AMD MI355X (gfx950)."""
