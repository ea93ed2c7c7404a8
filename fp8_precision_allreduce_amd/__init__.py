"""FP8 low-precision collective compute for MI355X (gfx950)."""
