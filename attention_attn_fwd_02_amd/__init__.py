"""MI355X-native fused attention forward (gfx950 HIP kernels behind a C ABI)."""
