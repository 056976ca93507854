"""int4 group-wise (g=64) compressed decode path for MI355X (gfx950)."""
