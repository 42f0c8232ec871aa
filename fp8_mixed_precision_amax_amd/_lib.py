"""ctypes binding of libfp8linear.so (the C ABI in include/fp8_linear.h).

Argument marshalling only: every step of the FP8 linear runs in the HIP
library.  torch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream().cuda_stream``).  If the library has not been
built this module raises on import: there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8linear.so")

# enums (mirror include/fp8_linear.h)
E4M3, E5M2 = 0, 1
SCALE_TENSOR, SCALE_1x128, SCALE_128x128 = 0, 1, 2
RECIPE_TENSOR, RECIPE_BLOCK = 0, 1
LAYOUT_ROW, LAYOUT_COL = 1, 2
STATUS = {0: "FP8_OK", 1: "FP8_ERR_NULL", 2: "FP8_ERR_SHAPE", 3: "FP8_ERR_ALIGN", 4: "FP8_ERR_ENUM",
          5: "FP8_ERR_WORKSPACE", 6: "FP8_ERR_CACHE_EMPTY", 7: "FP8_ERR_CACHE_MISMATCH", 8: "FP8_ERR_HIP",
          9: "FP8_ERR_UNIMPLEMENTED"}
NOALLOC_SCRATCH_BYTES = 8 << 20   # FP8_NOALLOC_SCRATCH_BYTES

# every symbol include/fp8_linear.h declares
EXPORTS = [
    "fp8_quantize_workspace_bytes", "fp8_quantize", "fp8_quantize_from_amax",
    "fp8_quantize_delayed_workspace_bytes", "fp8_quantize_delayed", "fp8_gemm_workspace_bytes",
    "fp8_gemm", "fp8_gemm_amax",
    "fp8_wcache_create", "fp8_wcache_invalidate", "fp8_wcache_valid", "fp8_wcache_fills",
    "fp8_wcache_destroy", "fp8_linear_workspace_bytes", "fp8_linear_fwd", "fp8_linear_bwd",
    "fp8_gelu", "fp8_dgelu", "fp8_quantize_gelu", "fp8_quantize_dgelu", "fp8_linear_fwd_gelu",
    "fp8_linear_bwd_dgelu", "fp8_linear_fwd_noalloc", "fp8_gemm_gelu_amax", "fp8_quantize_gelu_from_amax",
    "fp8_mlp_workspace_bytes", "fp8_mlp_fwd", "fp8_bf16_gemm_workspace_bytes", "fp8_bf16_gemm",
    "fp8_bf16_linear_workspace_bytes", "fp8_bf16_linear_fwd", "fp8_bf16_linear_bwd",
    "fp8_status_string", "fp8_last_error", "fp8_version",
]


class Fp8Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class QTensorC(ctypes.Structure):
    _fields_ = [("q_row", ctypes.c_void_p), ("q_col", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("scale_inv", ctypes.c_void_p),
                ("scale_col", ctypes.c_void_p), ("scale_inv_col", ctypes.c_void_p),
                ("amax", ctypes.c_void_p)]


class GemmScaleC(ctypes.Structure):
    _fields_ = [("scale_inv", ctypes.c_void_p), ("group", ctypes.c_int64),
                ("stride_r", ctypes.c_int64), ("stride_kb", ctypes.c_int64)]


_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfp8linear.so is not built (run __graft_entry__.build() or "
                          "python fp8_mixed_precision_amax_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, U, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    QP = ctypes.POINTER(QTensorC)
    sig = {
        "fp8_quantize_workspace_bytes": (SZ, [I64, I64, I]),
        "fp8_quantize": (I, [P, I64, I64, I, I, U, QP, P, SZ, P]),
        "fp8_gemm_workspace_bytes": (SZ, [I64, I64, I64]),
        "fp8_gemm": (I, [P, I, GemmScaleC, P, I, GemmScaleC, I64, I64, I64, P, P, SZ, P]),
        "fp8_wcache_create": (I, [I64, I64, I, QP, ctypes.POINTER(P)]),
        "fp8_wcache_invalidate": (I, [P]),
        "fp8_wcache_valid": (I, [P]),
        "fp8_wcache_fills": (I64, [P]),
        "fp8_wcache_destroy": (None, [P]),
        "fp8_linear_workspace_bytes": (SZ, [I64, I64, I64, I]),
        "fp8_linear_fwd": (I, [P, P, I64, I64, I64, I, P, I, P, QP, QP, P, P, P, SZ, P]),
        "fp8_linear_bwd": (I, [P, I64, I64, I64, I, QP, P, QP, QP, P, P, P, P, P, SZ, P]),
        "fp8_quantize_from_amax": (I, [P, I64, I64, I, U, QP, P, P]),
        "fp8_quantize_delayed_workspace_bytes": (SZ, [I64, I64]),
        "fp8_quantize_delayed": (I, [P, I64, I64, I, U, QP, P, I64, P, SZ, P]),
        "fp8_gemm_amax": (I, [P, I, GemmScaleC, P, I, GemmScaleC, I64, I64, I64, P, P, P, SZ, P]),
        "fp8_gelu": (I, [P, P, I64, P]),
        "fp8_dgelu": (I, [P, P, P, I64, P]),
        "fp8_quantize_gelu": (I, [P, I64, I64, I, I, U, QP, P, SZ, P]),
        "fp8_quantize_dgelu": (I, [P, P, I64, I64, I, I, U, QP, P, SZ, P]),
        "fp8_linear_fwd_gelu": (I, [P, P, I64, I64, I64, I, P, I, P, QP, QP, P, P, SZ, P]),
        "fp8_linear_bwd_dgelu": (I, [P, P, I64, I64, I64, I, QP, P, QP, QP, P, P, P, P, SZ, P]),
        "fp8_linear_fwd_noalloc": (I, [P, P, I64, I64, I64, I, P, I, P, QP, QP, P, P, P]),
        "fp8_gemm_gelu_amax": (I, [P, I, GemmScaleC, P, I, GemmScaleC, I64, I64, I64, P, P, P, SZ, P]),
        "fp8_quantize_gelu_from_amax": (I, [P, I64, I64, I, U, QP, P, P]),
        "fp8_mlp_workspace_bytes": (SZ, [I64, I64, I64, I]),
        "fp8_bf16_gemm_workspace_bytes": (SZ, [I64, I64, I64]),
        "fp8_bf16_gemm": (I, [P, I, P, I, I64, I64, I64, P, P, SZ, P]),
        "fp8_bf16_linear_workspace_bytes": (SZ, [I64, I64, I64]),
        "fp8_bf16_linear_fwd": (I, [P, P, I64, I64, I64, P, P, SZ, P]),
        "fp8_bf16_linear_bwd": (I, [P, P, P, I64, I64, I64, P, P, P, SZ, P]),
        "fp8_mlp_fwd": (I, [P, P, P, I64, I64, I64, I, P, P, I, P, P, QP, QP, QP, QP, P, P, P, SZ, P]),
        "fp8_status_string": (ctypes.c_char_p, [I]),
        "fp8_last_error": (ctypes.c_char_p, []),
        "fp8_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status):
    if status != 0:
        raise Fp8Error(status, load().fp8_last_error().decode())
    return status
