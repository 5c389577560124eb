"""MI355X-native (gfx950) Q2_0 hot path: get_rows, decode mat-vec, prefill GEMM (F32, F16 or
BF16 activations, F32 results).

The computation lives in libq2_0.so (hand-written HIP, C ABI in include/q2_0.h);
``q2_0`` is its ctypes binding and ``synth`` the seeded synthetic-input generator.
Importing the package does not load the library; the first call does, and fails
loudly if it has not been built.
"""

from .q2_0 import (  # noqa: F401
    Q2_0_ACT_BF16, Q2_0_ACT_F16, Q2_0_ACT_F32, Q2_0_PREC_F16_MFMA, Q2_0_PREC_F32, Q2_0Error, q2_0_get_rows,
    q2_0_mul_mat, q2_0_mul_mat_group, q2_0_mul_mat_id, q2_0_mul_mat_vec, q2_0_mul_mat_vec_batch, q2_0_mul_mat_vec_group,
    q2_0_quantize, q2_0_repack_g128,
)
