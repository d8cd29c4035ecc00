"""Paged KV-cache single-token decode attention for AMD MI355X (gfx950)."""
