"""Dequantize-fused low-bit matrix-vector / matrix-matrix products and a fused
greedy (argmax) head for AMD MI355X (gfx950)."""
