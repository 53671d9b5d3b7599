"""Attention over an FP8 (OCP e4m3fn) KV cache on MI355X (gfx950)."""
