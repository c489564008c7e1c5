"""ctypes binding of libgemm's C ABI (argument marshalling only).

The functions here have the names and argument order of ``include/libgemm.h``
and take device pointers as integers.  Every computation happens in the HIP
kernels of ``libgemm.so``; if that library is missing or cannot be loaded this
module raises instead of computing anything another way.

``torch`` is imported first so that the process has one HIP runtime: torch's
own ``libamdhip64`` carries the same soname as the system one, so the loader
resolves libgemm's dependency to the already-loaded copy and device pointers
and streams from torch are valid in libgemm calls.
"""
import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libgemm links against)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm.so")

ROW_MAJOR, COL_MAJOR = 0, 1
DTYPE_SAME, DTYPE_F32 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
F8_E4M3, F8_E5M2 = 0, 1
MX_E4M3, MX_E5M2, MX_E2M3, MX_E3M2, MX_E2M1 = 0, 1, 2, 3, 4
MX_FORMAT = {"e4m3": MX_E4M3, "e5m2": MX_E5M2, "e2m3": MX_E2M3, "e3m2": MX_E3M2, "e2m1": MX_E2M1}
OUTPUT_F32, OUTPUT_BF16, OUTPUT_F16 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4
# gemm_test_switches flags
TEST_FORCE_GENERAL, TEST_NO_SPLITK, TEST_FORCE_STREAMK, TEST_F32_VALU = 1, 2, 4, 8
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def library() -> ctypes.CDLL:
    """The loaded libgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libgemm.so not found at {LIB_PATH}; build it with "
                "`python -m dense_gemm_optimisation_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        i64, f32, vp, i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
        common = [i64, i64, i64, f32, vp, i64, i32, vp, i64, i32, f32, vp, i64, i32]
        lib.gemm_f32.argtypes = common + [i64, i64, i64, i64, vp]
        lib.gemm_f32.restype = i32
        for name in ("gemm_bf16", "gemm_f16"):
            fn = getattr(lib, name)
            fn.argtypes = common + [i32, i64, i64, i64, i64, vp]
            fn.restype = i32
        lib.gemm_status_string.argtypes = [i32]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_abi_version.restype = i32
        lib.gemm_f32_bias_act.argtypes = common + [i64, i64, i64, i64, vp, i64, i32, vp]
        lib.gemm_f32_bias_act.restype = i32
        for name in ("gemm_bf16_bias_act", "gemm_f16_bias_act"):
            fn = getattr(lib, name)
            fn.argtypes = common + [i32, i64, i64, i64, i64, vp, i64, i32, vp]
            fn.restype = i32
        lib.gemm_kernel_name.argtypes = [i32] + common + [i32, i64, i64, i64, i64]
        lib.gemm_kernel_name.restype = ctypes.c_char_p
        f8 = [i64, i64, i64, f32, vp, i64, i32, i32, vp, i64, i32, i32, f32, vp, i64, i32, i32,
              i64, i64, i64, i64]
        lib.gemm_f8.argtypes = f8 + [vp]
        lib.gemm_f8.restype = i32
        lib.gemm_f8_kernel_name.argtypes = f8
        lib.gemm_f8_kernel_name.restype = ctypes.c_char_p
        mx = [i64, i64, i64, f32, vp, i64, i32, vp, i64, vp, i64, i32, vp, i64, f32, vp, i64,
              i32, i32, i64, i64, i64, i64, i64, i64]
        lib.gemm_mx.argtypes = mx + [vp]
        lib.gemm_mx.restype = i32
        lib.gemm_mx_kernel_name.argtypes = mx
        lib.gemm_mx_kernel_name.restype = ctypes.c_char_p
        sz = ctypes.c_size_t
        lib.gemm_f8_ws.argtypes = f8 + [vp, sz, vp]
        lib.gemm_f8_ws.restype = i32
        lib.gemm_f8_kernel_name_ws.argtypes = f8 + [vp, sz]
        lib.gemm_f8_kernel_name_ws.restype = ctypes.c_char_p
        lib.gemm_mx_ws.argtypes = mx + [vp, sz, vp]
        lib.gemm_mx_ws.restype = i32
        lib.gemm_mx_kernel_name_ws.argtypes = mx + [vp, sz]
        lib.gemm_mx_kernel_name_ws.restype = ctypes.c_char_p
        lib.gemm_workspace_size.argtypes = []
        lib.gemm_workspace_size.restype = sz
        for name in ("gemm_bf16_ws", "gemm_f16_ws"):
            fn = getattr(lib, name)
            fn.argtypes = common + [i32, i64, i64, i64, i64, vp, sz, vp]
            fn.restype = i32
        lib.gemm_f32_valu.argtypes = common + [i64, i64, i64, i64, vp]
        lib.gemm_f32_valu.restype = i32
        lib.gemm_test_switches.argtypes = [i32]
        lib.gemm_test_switches.restype = i32
        lib.gemm_bf16_noalloc.argtypes = common + [i32, i64, i64, i64, i64, vp]
        lib.gemm_bf16_noalloc.restype = i32
        lib.gemm_f32_ws.argtypes = common + [i64, i64, i64, i64, vp, sz, vp]
        lib.gemm_f32_ws.restype = i32
        lib.gemm_kernel_name_ws.argtypes = [i32] + common + [i32, i64, i64, i64, i64, vp, sz]
        lib.gemm_kernel_name_ws.restype = ctypes.c_char_p
        quant = [i64, i64, i64, f32, vp, i64, i32, vp, i64, i32, vp, i64, i32, i32, f32, i64, i64,
                 i64, i64, vp, i64, i32, vp]
        for name in ("gemm_bf16_quant", "gemm_f16_quant"):
            fn = getattr(lib, name)
            fn.argtypes = quant
            fn.restype = i32
        lib.gemm_kernel_name_quant.argtypes = [i32, i64, i64, i64, f32, vp, i64, i32, vp, i64, i32,
                                               vp, i64, i32, i32, i64, i64, i64, i64]
        lib.gemm_kernel_name_quant.restype = ctypes.c_char_p
        lib.gemm_f32_bf16x3_workspace_size.argtypes = [i64, i64, i64, i64]
        lib.gemm_f32_bf16x3_workspace_size.restype = sz
        lib.gemm_f32_bf16x3.argtypes = common + [i64, i64, i64, i64, vp, sz, vp]
        lib.gemm_f32_bf16x3.restype = i32
        lib.gemm_kernel_name_bf16x3.argtypes = common + [i64, i64, i64, i64, vp, sz]
        lib.gemm_kernel_name_bf16x3.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().gemm_status_string(status).decode()


def abi_version() -> int:
    return library().gemm_abi_version()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _check(status, name, raise_on_error):
    if raise_on_error and status != OK:
        raise GemmError(status, name)
    return status


def gemm_f32(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
             batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None, raise_on_error=True):
    """C <- alpha*op(A)*op(B) + beta*C in fp32; A, B, C are device addresses (int)."""
    st = library().gemm_f32(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                            order_c, batch, stride_a, stride_b, stride_c, _stream(stream))
    return _check(st, "gemm_f32", raise_on_error)


def gemm_f32_valu(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                  batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None, raise_on_error=True):
    """gemm_f32 on the vector-ALU kernel (register-tiled fused multiply-adds)."""
    st = library().gemm_f32_valu(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                                 order_c, batch, stride_a, stride_b, stride_c, _stream(stream))
    return _check(st, "gemm_f32_valu", raise_on_error)


def test_switches(flags: int) -> int:
    """Set the process-wide kernel-choice overrides (TEST_* flags, 0 clears
    them); returns the previous set.  For tests only."""
    return library().gemm_test_switches(int(flags))


def gemm_bf16(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
              c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None,
              raise_on_error=True):
    """bf16 inputs, fp32 accumulation, bf16 (DTYPE_SAME) or fp32 (DTYPE_F32) C."""
    st = library().gemm_bf16(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                             order_c, c_dtype, batch, stride_a, stride_b, stride_c,
                             _stream(stream))
    return _check(st, "gemm_bf16", raise_on_error)


def gemm_f16(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
             c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None,
             raise_on_error=True):
    """fp16 inputs, fp32 accumulation, fp16 (DTYPE_SAME) or fp32 (DTYPE_F32) C."""
    st = library().gemm_f16(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                            order_c, c_dtype, batch, stride_a, stride_b, stride_c,
                            _stream(stream))
    return _check(st, "gemm_f16", raise_on_error)


def gemm_f32_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                      batch=1, stride_a=0, stride_b=0, stride_c=0, bias=0, stride_bias=0,
                      act=ACT_NONE, stream=None, raise_on_error=True):
    """C <- act(alpha*op(A)*op(B) + beta*C + bias) in fp32; bias is a device
    address of N floats per batch entry (0 for none)."""
    st = library().gemm_f32_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C,
                                     ldc, order_c, batch, stride_a, stride_b, stride_c, bias,
                                     stride_bias, act, _stream(stream))
    return _check(st, "gemm_f32_bias_act", raise_on_error)


def gemm_bf16_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                       c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, bias=0,
                       stride_bias=0, act=ACT_NONE, stream=None, raise_on_error=True):
    """bf16 inputs with the fused bias/activation epilogue (bias in bf16)."""
    st = library().gemm_bf16_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C,
                                      ldc, order_c, c_dtype, batch, stride_a, stride_b, stride_c,
                                      bias, stride_bias, act, _stream(stream))
    return _check(st, "gemm_bf16_bias_act", raise_on_error)


def gemm_f16_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                      c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, bias=0,
                      stride_bias=0, act=ACT_NONE, stream=None, raise_on_error=True):
    """fp16 inputs with the fused bias/activation epilogue (bias in fp16)."""
    st = library().gemm_f16_bias_act(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C,
                                     ldc, order_c, c_dtype, batch, stride_a, stride_b, stride_c,
                                     bias, stride_bias, act, _stream(stream))
    return _check(st, "gemm_f16_bias_act", raise_on_error)


def gemm_f8(M, N, K, alpha, A, lda, order_a, format_a, B, ldb, order_b, format_b, beta, C, ldc,
            order_c, type_c, batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None,
            raise_on_error=True):
    """8-bit float inputs (F8_E4M3 / F8_E5M2 per operand), fp32 accumulation,
    C of type OUTPUT_F32, OUTPUT_BF16 or OUTPUT_F16."""
    st = library().gemm_f8(M, N, K, alpha, A, lda, order_a, format_a, B, ldb, order_b, format_b,
                           beta, C, ldc, order_c, type_c, batch, stride_a, stride_b, stride_c,
                           _stream(stream))
    return _check(st, "gemm_f8", raise_on_error)


def gemm_f8_ws(M, N, K, alpha, A, lda, order_a, format_a, B, ldb, order_b, format_b, beta, C,
               ldc, order_c, type_c, batch, stride_a, stride_b, stride_c, workspace,
               workspace_bytes, stream=None, raise_on_error=True):
    """gemm_f8 with a caller workspace (stream-K schedule where it pays)."""
    st = library().gemm_f8_ws(M, N, K, alpha, A, lda, order_a, format_a, B, ldb, order_b,
                              format_b, beta, C, ldc, order_c, type_c, batch, stride_a, stride_b,
                              stride_c, workspace, workspace_bytes, _stream(stream))
    return _check(st, "gemm_f8_ws", raise_on_error)


def f8_kernel_name(M, N, K, alpha, A, lda, order_a, format_a, B, ldb, order_b, format_b, beta, C,
                   ldc, order_c, type_c, batch=1, stride_a=0, stride_b=0, stride_c=0,
                   workspace=None, workspace_bytes=0):
    """The kernel gemm_f8 (gemm_f8_ws with a workspace) would launch for these
    arguments (see kernel_name)."""
    lib = library()
    if workspace is None:
        name = lib.gemm_f8_kernel_name(M, N, K, alpha, A, lda, order_a, format_a, B, ldb,
                                       order_b, format_b, beta, C, ldc, order_c, type_c, batch,
                                       stride_a, stride_b, stride_c)
    else:
        name = lib.gemm_f8_kernel_name_ws(M, N, K, alpha, A, lda, order_a, format_a, B, ldb,
                                          order_b, format_b, beta, C, ldc, order_c, type_c,
                                          batch, stride_a, stride_b, stride_c, workspace,
                                          workspace_bytes)
    return None if name is None else name.decode()


def gemm_mx(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb, format_b, scale_b, ldsb,
            beta, C, ldc, order_c, type_c, batch=1, stride_a=0, stride_b=0, stride_scale_a=0,
            stride_scale_b=0, stride_c=0, stream=None, raise_on_error=True):
    """Block-scaled inputs (MX_* formats, E8M0 scales per 32 elements along
    K), A row-major and B column-major (both contiguous along K), output
    type_c (OUTPUT_*).  Device addresses as integers."""
    st = library().gemm_mx(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb, format_b,
                           scale_b, ldsb, beta, C, ldc, order_c, type_c, batch, stride_a, stride_b,
                           stride_scale_a, stride_scale_b, stride_c, _stream(stream))
    return _check(st, "gemm_mx", raise_on_error)


def gemm_mx_ws(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb, format_b, scale_b, ldsb,
               beta, C, ldc, order_c, type_c, batch, stride_a, stride_b, stride_scale_a,
               stride_scale_b, stride_c, workspace, workspace_bytes, stream=None,
               raise_on_error=True):
    """gemm_mx with a caller workspace (stream-K schedule where it pays)."""
    st = library().gemm_mx_ws(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb, format_b,
                              scale_b, ldsb, beta, C, ldc, order_c, type_c, batch, stride_a,
                              stride_b, stride_scale_a, stride_scale_b, stride_c, workspace,
                              workspace_bytes, _stream(stream))
    return _check(st, "gemm_mx_ws", raise_on_error)


def mx_kernel_name(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb, format_b, scale_b,
                   ldsb, beta, C, ldc, order_c, type_c, batch=1, stride_a=0, stride_b=0,
                   stride_scale_a=0, stride_scale_b=0, stride_c=0, workspace=None,
                   workspace_bytes=0):
    """The kernel gemm_mx (gemm_mx_ws with a workspace) would launch for these
    arguments (None if invalid)."""
    lib = library()
    if workspace is None:
        name = lib.gemm_mx_kernel_name(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb,
                                       format_b, scale_b, ldsb, beta, C, ldc, order_c, type_c,
                                       batch, stride_a, stride_b, stride_scale_a, stride_scale_b,
                                       stride_c)
    else:
        name = lib.gemm_mx_kernel_name_ws(M, N, K, alpha, A, lda, format_a, scale_a, ldsa, B, ldb,
                                          format_b, scale_b, ldsb, beta, C, ldc, order_c, type_c,
                                          batch, stride_a, stride_b, stride_scale_a,
                                          stride_scale_b, stride_c, workspace, workspace_bytes)
    return None if name is None else name.decode()


def workspace_size() -> int:
    """Bytes of workspace that let the *_ws entry points use every schedule."""
    return library().gemm_workspace_size()


def gemm_f32_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                batch=1, stride_a=0, stride_b=0, stride_c=0, workspace=0, workspace_bytes=0,
                stream=None, raise_on_error=True):
    """gemm_f32 with a device workspace (address, bytes) for the stream-K schedule."""
    st = library().gemm_f32_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                               order_c, batch, stride_a, stride_b, stride_c, workspace,
                               workspace_bytes, _stream(stream))
    return _check(st, "gemm_f32_ws", raise_on_error)


def gemm_quant(in_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
               c_format, c_scale=1.0, batch=1, stride_a=0, stride_b=0, stride_c=0, bias=None,
               stride_bias=0, act=0, stream=None, raise_on_error=True):
    """gemm_bf16_quant / gemm_f16_quant: the fused epilogue, scaled by c_scale
    and stored as 8-bit floats of c_format ("e4m3" or "e5m2")."""
    fn = library().gemm_bf16_quant if in_dtype == "bf16" else library().gemm_f16_quant
    st = fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
            _F8_FORMAT[c_format], c_scale, batch, stride_a, stride_b, stride_c, bias, stride_bias,
            act, _stream(stream))
    return _check(st, "gemm_quant", raise_on_error)


def kernel_name_quant(in_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, C, ldc, order_c,
                      c_format, batch=1, stride_a=0, stride_b=0, stride_c=0):
    """The kernel gemm_bf16_quant / gemm_f16_quant would launch, or None."""
    name = library().gemm_kernel_name_quant(_INPUT[in_dtype], M, N, K, alpha, A, lda, order_a, B,
                                            ldb, order_b, C, ldc, order_c, _F8_FORMAT[c_format],
                                            batch, stride_a, stride_b, stride_c)
    return None if name is None else name.decode()


def bf16x3_workspace_size(M, N, K, batch=1):
    """Bytes of workspace gemm_f32_bf16x3 needs for these sizes."""
    return library().gemm_f32_bf16x3_workspace_size(M, N, K, batch)


def gemm_f32_bf16x3(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                    batch=1, stride_a=0, stride_b=0, stride_c=0, workspace=0, workspace_bytes=0,
                    stream=None, raise_on_error=True):
    """fp32 GEMM as three bf16 products of split operands; the workspace
    (address, bytes) receives the split copies."""
    st = library().gemm_f32_bf16x3(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C,
                                   ldc, order_c, batch, stride_a, stride_b, stride_c, workspace,
                                   workspace_bytes, _stream(stream))
    return _check(st, "gemm_f32_bf16x3", raise_on_error)


def kernel_name_bf16x3(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                       batch=1, stride_a=0, stride_b=0, stride_c=0, workspace=0,
                       workspace_bytes=0):
    """The bf16 kernel gemm_f32_bf16x3 would run ("scale"/"" when nothing is
    multiplied, None for invalid arguments); host only."""
    name = library().gemm_kernel_name_bf16x3(M, N, K, alpha, A, lda, order_a, B, ldb, order_b,
                                             beta, C, ldc, order_c, batch, stride_a, stride_b,
                                             stride_c, workspace, workspace_bytes)
    return None if name is None else name.decode()


def gemm_bf16_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                 c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, workspace=0,
                 workspace_bytes=0, stream=None, raise_on_error=True):
    """gemm_bf16 with a device workspace (address, bytes) for the stream-K schedule."""
    st = library().gemm_bf16_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                                order_c, c_dtype, batch, stride_a, stride_b, stride_c, workspace,
                                workspace_bytes, _stream(stream))
    return _check(st, "gemm_bf16_ws", raise_on_error)


def gemm_bf16_noalloc(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                      c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0,
                      stream=None, raise_on_error=True):
    """gemm_bf16_ws without a caller workspace: the library's per-device scratch."""
    st = library().gemm_bf16_noalloc(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C,
                                     ldc, order_c, c_dtype, batch, stride_a, stride_b, stride_c,
                                     _stream(stream))
    return _check(st, "gemm_bf16_noalloc", raise_on_error)


def gemm_f16_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, workspace=0,
                workspace_bytes=0, stream=None, raise_on_error=True):
    """gemm_f16 with a device workspace (address, bytes) for the stream-K schedule."""
    st = library().gemm_f16_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                               order_c, c_dtype, batch, stride_a, stride_b, stride_c, workspace,
                               workspace_bytes, _stream(stream))
    return _check(st, "gemm_f16_ws", raise_on_error)


_F8_FORMAT = {"e4m3": F8_E4M3, "e5m2": F8_E5M2}
_OUTPUT = {"f32": OUTPUT_F32, "bf16": OUTPUT_BF16, "f16": OUTPUT_F16}

_ENTRY = {"f32": gemm_f32, "bf16": gemm_bf16, "f16": gemm_f16}
_ENTRY_EPI = {"f32": gemm_f32_bias_act, "bf16": gemm_bf16_bias_act, "f16": gemm_f16_bias_act}
_INPUT = {"f32": 0, "bf16": 1, "f16": 2}


def kernel_name(in_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, b_dtype=None,
                out_dtype=None, workspace=None, workspace_bytes=0):
    """The kernel the GEMM call with these arguments would launch ("" for an
    empty problem, None for invalid arguments); host only, no GPU needed.
    For 8-bit inputs ("e4m3"/"e5m2") b_dtype and out_dtype name B's format
    and C's type, as in gemm(); a workspace asks about the workspace entry
    points."""
    if in_dtype in _F8_FORMAT:
        return f8_kernel_name(M, N, K, alpha, A, lda, order_a, _F8_FORMAT[in_dtype], B, ldb,
                              order_b, _F8_FORMAT[b_dtype or in_dtype], beta, C, ldc, order_c,
                              _OUTPUT[out_dtype], batch, stride_a, stride_b, stride_c, workspace,
                              workspace_bytes)
    if workspace is not None:
        name = library().gemm_kernel_name_ws(_INPUT[in_dtype], M, N, K, alpha, A, lda, order_a, B,
                                             ldb, order_b, beta, C, ldc, order_c, c_dtype, batch,
                                             stride_a, stride_b, stride_c, workspace,
                                             workspace_bytes)
        return None if name is None else name.decode()
    name = library().gemm_kernel_name(_INPUT[in_dtype], M, N, K, alpha, A, lda, order_a, B, ldb,
                                      order_b, beta, C, ldc, order_c, c_dtype, batch, stride_a,
                                      stride_b, stride_c)
    return None if name is None else name.decode()


def gemm(in_dtype, M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
         c_dtype=DTYPE_SAME, batch=1, stride_a=0, stride_b=0, stride_c=0, stream=None,
         raise_on_error=True, bias=None, stride_bias=0, act=ACT_NONE, b_dtype=None,
         out_dtype=None, workspace=None, workspace_bytes=0, valu=False):
    """Dispatch on the input type name ("f32", "bf16", "f16", or the 8-bit
    "e4m3"/"e5m2" with B's format in b_dtype (default: A's) and C's type
    name in out_dtype); a bias address or an activation selects the
    fused-epilogue entry point (not offered for 8-bit inputs); a workspace
    address (no epilogue) selects the workspace entry point;
    valu=True (fp32, no epilogue, no workspace) selects gemm_f32_valu."""
    if valu:
        if in_dtype != "f32" or workspace is not None or bias is not None or act != ACT_NONE:
            raise ValueError("gemm_f32_valu takes fp32 inputs without workspace or epilogue")
        return gemm_f32_valu(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                             order_c, batch, stride_a, stride_b, stride_c, stream, raise_on_error)
    if workspace is not None:
        if bias is not None or act != ACT_NONE:
            raise ValueError("the workspace entry points have no fused epilogue")
        if in_dtype in _F8_FORMAT:
            return gemm_f8_ws(M, N, K, alpha, A, lda, order_a, _F8_FORMAT[in_dtype], B, ldb,
                              order_b, _F8_FORMAT[b_dtype or in_dtype], beta, C, ldc, order_c,
                              _OUTPUT[out_dtype], batch, stride_a, stride_b, stride_c, workspace,
                              workspace_bytes, stream, raise_on_error)
        if in_dtype == "f32":
            return gemm_f32_ws(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc,
                               order_c, batch, stride_a, stride_b, stride_c, workspace,
                               workspace_bytes, stream, raise_on_error)
        fn = gemm_bf16_ws if in_dtype == "bf16" else gemm_f16_ws
        return fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c, c_dtype,
                  batch, stride_a, stride_b, stride_c, workspace, workspace_bytes, stream,
                  raise_on_error)
    if in_dtype in _F8_FORMAT:
        if bias is not None or act != ACT_NONE:
            raise ValueError("8-bit inputs have no fused-epilogue entry point")
        return gemm_f8(M, N, K, alpha, A, lda, order_a, _F8_FORMAT[in_dtype], B, ldb, order_b,
                       _F8_FORMAT[b_dtype or in_dtype], beta, C, ldc, order_c, _OUTPUT[out_dtype],
                       batch, stride_a, stride_b, stride_c, stream, raise_on_error)
    if bias is not None or act != ACT_NONE:
        fn = _ENTRY_EPI[in_dtype]
        if in_dtype == "f32":
            return fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                      batch, stride_a, stride_b, stride_c, bias or 0, stride_bias, act, stream,
                      raise_on_error)
        return fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                  c_dtype, batch, stride_a, stride_b, stride_c, bias or 0, stride_bias, act,
                  stream, raise_on_error)
    fn = _ENTRY[in_dtype]
    if in_dtype == "f32":
        return fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c,
                  batch, stride_a, stride_b, stride_c, stream, raise_on_error)
    return fn(M, N, K, alpha, A, lda, order_a, B, ldb, order_b, beta, C, ldc, order_c, c_dtype,
              batch, stride_a, stride_b, stride_c, stream, raise_on_error)


def _matrix_layout(t):
    """(order, ld) of a 2-D strided view, or None if it is neither row- nor column-major."""
    r, c = t.shape[-2], t.shape[-1]
    sr, sc = t.stride(-2), t.stride(-1)
    if sc == 1 or c == 1:
        return ROW_MAJOR, max(sr if r > 1 else c, c, 1)
    if sr == 1 or r == 1:
        return COL_MAJOR, max(sc if c > 1 else r, r, 1)
    return None


_TORCH_IN = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def matmul(a, b, c=None, alpha=1.0, beta=0.0, out_dtype=None, stream=None, bias=None,
           act=ACT_NONE):
    """C = act(alpha*a@b + beta*c + bias) on torch CUDA tensors (2-D, or 3-D batched).

    ``a`` (..., M, K) and ``b`` (..., K, N) may be row- or column-major views;
    a 3-D operand with batch stride 0 (an expanded view) is shared across the
    batch.  ``bias`` (optional) is a contiguous (N,) or (batch, N) tensor of
    the input type; ``act`` is ACT_NONE, ACT_RELU or ACT_GELU.  Returns ``c``
    (allocated when None).  Only marshalling happens here.
    """
    if a.dtype != b.dtype or a.dtype not in _TORCH_IN:
        raise TypeError("a and b must share one of float32, bfloat16, float16")
    in_dtype = _TORCH_IN[a.dtype]
    batched = a.dim() == 3 or b.dim() == 3
    M, K = a.shape[-2], a.shape[-1]
    N = b.shape[-1]
    if b.shape[-2] != K:
        raise ValueError("inner dimensions differ")
    batch = max(a.shape[0] if a.dim() == 3 else 1, b.shape[0] if b.dim() == 3 else 1)
    if out_dtype is None:
        out_dtype = a.dtype if c is None else c.dtype
    if in_dtype == "f32" and out_dtype != torch.float32:
        raise TypeError("fp32 inputs give fp32 output")
    if out_dtype not in (a.dtype, torch.float32):
        raise TypeError("output must be the input type or float32")
    if c is None:
        shape = (batch, M, N) if batched else (M, N)
        c = torch.empty(shape, dtype=out_dtype, device=a.device)
        if beta != 0.0:
            raise ValueError("beta != 0 needs c")
    lay = [_matrix_layout(t) for t in (a, b, c)]
    if None in lay:
        raise ValueError("operands must be row- or column-major (unit stride in one dimension)")

    def bstride(t):
        return t.stride(0) if t.dim() == 3 and t.shape[0] > 1 else 0

    c_dtype = DTYPE_SAME if (out_dtype == a.dtype) else DTYPE_F32
    bias_ptr, bias_stride = None, 0
    if bias is not None:
        if bias.dtype != a.dtype or bias.shape[-1] != N or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous (N,) or (batch, N) tensor of the input type")
        bias_ptr = bias.data_ptr()
        bias_stride = N if (bias.dim() == 2 and bias.shape[0] > 1) else 0
    gemm(in_dtype, M, N, K, alpha, a.data_ptr(), lay[0][1], lay[0][0], b.data_ptr(), lay[1][1],
         lay[1][0], beta, c.data_ptr(), lay[2][1], lay[2][0], c_dtype, batch, bstride(a),
         bstride(b), bstride(c) if batch > 1 else 0, stream, bias=bias_ptr,
         stride_bias=bias_stride, act=act)
    return c
