"""CPU oracle for the W4A16 weight-only quantized GEMM (test infrastructure only).

Only the tests, the build entry point's smoke check and the bench's CPU-baseline leg may
import this package.  It shares no code with the HIP library under
weight_only_quantized_gemm_amd/ and never imports it.
"""
