"""Group-wise weight-only 3/4-bit quantization and fused dequantize-GEMV/GEMM for MI355X (gfx950)."""
