"""MI355X-native fp16 GEMM C = A * B^T (fp32 accumulate, fp16 out)."""
