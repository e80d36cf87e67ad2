"""CPU oracle for block-scaled FP4 quantization and FP4 GEMM.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the GPU product path never does.
"""
