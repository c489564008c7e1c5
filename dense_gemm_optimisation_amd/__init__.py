"""Dense GEMM for AMD Instinct MI355X (gfx950).

C = alpha*A*B + beta*C with fp32 inputs on the vector ALUs and bf16/fp16
inputs on the matrix cores (fp32 accumulation).  The computation lives in the
HIP kernels of ``libgemm.so`` behind the C ABI declared in
``include/libgemm.h``; this package is its Python binding and build script.
"""
from .binding import (COL_MAJOR, DTYPE_F32, DTYPE_SAME, ERR_HIP, ERR_INVALID_ARG,  # noqa: F401
                      ERR_UNSUPPORTED, OK, ROW_MAJOR, GemmError, abi_version, gemm, gemm_bf16,
                      gemm_f16, gemm_f32, library, matmul, status_string)
