"""NVFP4 weight x bf16 activation products on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI declared in
include/nvfp4.h (library libnvfp4.so, next to this file).  The Python
functions in `binding` only marshal torch device tensors into that ABI.
"""
