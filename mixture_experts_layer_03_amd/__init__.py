"""MI355X-native MoE expert block: router, permutation, grouped SwiGLU FFN,
combine, and their backward, as hand-written HIP kernels behind a C ABI."""
