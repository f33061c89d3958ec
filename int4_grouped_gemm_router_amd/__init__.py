"""MI355X-native int4 grouped-GEMM mixture-of-experts layer (HIP, gfx950)."""
