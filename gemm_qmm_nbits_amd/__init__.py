"""Fused low-bit dequantize-matmul for MI355X (gfx950)."""
