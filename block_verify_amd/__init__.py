"""MI355X-native block-verify speculative decoding (gfx950 HIP kernels behind a C ABI)."""
