"""Block-scaled low-precision MoE quantization and grouped expert GEMM for MI355X (gfx950).

The compute path is the HIP library ``libbsp.so`` behind the C ABI declared in
``include/bsp.h``; :mod:`block_scaled_precision_token_amd.ops` is a thin
binding over it.  The library is loaded on first use; calling an op without it
raises instead of falling back to anything else.
"""
__version__ = "0.1.0"
