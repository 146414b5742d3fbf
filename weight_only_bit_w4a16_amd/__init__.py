"""W4A16 dequantise-GEMM for MI355X (gfx950).  Binding filled in below."""
