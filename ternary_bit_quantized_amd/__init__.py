"""MI355X-native Q2_0 x F32 hot path: get_rows, decode mat-vec, prefill GEMM."""
