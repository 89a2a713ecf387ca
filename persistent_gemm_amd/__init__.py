"""persistent_gemm_amd: a Stream-K GEMM for MI355X (gfx950) behind a small C ABI."""
