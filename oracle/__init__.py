"""CPU oracle for the NVFP4 weight x bf16 activation product (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  The GPU library never imports it and it never imports the GPU
library.
"""
from .oracle import (  # noqa: F401
    build, e2m1, e4m3, bf16_to_f64, dequant, gemm, route, group, silu, moe, max_threads, quantize, mx_from_nvfp4, mx_from_bf16, mx_gemm,
)
