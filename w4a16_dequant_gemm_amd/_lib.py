"""ctypes view of ``libw4a16.so`` (the C ABI declared in ``include/w4a16.h``).

Only symbol loading and prototypes live here.  Loading never touches the GPU, so the
CPU test-suite can check exports and host-side argument validation.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_ALIGN, ERR_DTYPE, ERR_SCHEME, ERR_HIP, ERR_PATH, ERR_SCRATCH = \
    -1, -2, -3, -4, -5, -6, -7, -8, -9
F16, BF16 = 0, 1
ASYM, SYM = 0, 1
PATH_AUTO, PATH_GEMV, PATH_SKINNY, PATH_PREFILL = 0, 1, 2, 3
PATH_NAMES = {PATH_GEMV: "gemv", PATH_SKINNY: "skinny", PATH_PREFILL: "prefill"}

class LinearItem(ctypes.Structure):
    """``w4a16_linear_item`` of the C ABI."""
    _fields_ = [("X", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("group_size", ctypes.c_int64), ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("Y", ctypes.c_void_p)]


_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib().w4a16_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else msg)


def lib() -> ctypes.CDLL:
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m w4a16_dequant_gemm_amd.build` "
            "(the W4A16 layer has no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.w4a16_abi_version.restype = i32
    L.w4a16_abi_version.argtypes = []
    L.w4a16_strerror.restype = ctypes.c_char_p
    L.w4a16_strerror.argtypes = [i32]
    L.w4a16_quantize_pack.restype = i32
    L.w4a16_quantize_pack.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, vp]
    L.w4a16_linear.restype = i32
    L.w4a16_linear.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.w4a16_linear_ex.restype = i32
    L.w4a16_linear_ex.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    L.w4a16_select_path.restype = i32
    L.w4a16_select_path.argtypes = [i64, i64, i64, i64, i32]
    L.w4a16_linear_workspace.restype = i64
    L.w4a16_linear_workspace.argtypes = [i64, i64, i64, i64, i32]
    L.w4a16_linear_ws.restype = i32
    L.w4a16_linear_ws.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.w4a16_linear_batch.restype = i32
    L.w4a16_linear_batch.argtypes = [ctypes.POINTER(LinearItem), i32, i32, vp]
    L.w4a16_linear_ws_noalloc.restype = i32
    L.w4a16_linear_ws_noalloc.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.w4a16_w8a16_quantize_pack.restype = i32
    L.w4a16_w8a16_quantize_pack.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, vp]
    L.w4a16_w8a16_linear.restype = i32
    L.w4a16_w8a16_linear.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.w4a16_w8a16_linear_ex.restype = i32
    L.w4a16_w8a16_linear_ex.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    L.w4a16_w8a16_select_path.restype = i32
    L.w4a16_w8a16_select_path.argtypes = [i64, i64, i64, i64, i32]
    L.w4a16_dequantize.restype = i32
    L.w4a16_dequantize.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp]
    L.w4a16_gptq_hessian.restype = i32
    L.w4a16_gptq_hessian.argtypes = [vp, i32, i64, i64, vp, i32, vp]
    L.w4a16_gptq_factor.restype = i32
    L.w4a16_gptq_factor.argtypes = [vp, i64, ctypes.c_double, vp, vp]
    L.w4a16_awq_workspace.restype = i64
    L.w4a16_awq_workspace.argtypes = [i64, i64, i64]
    L.w4a16_awq_stats.restype = i32
    L.w4a16_awq_stats.argtypes = [vp, i32, i64, i64, vp, vp]
    L.w4a16_awq_search.restype = i32
    L.w4a16_awq_search.argtypes = [vp, i64, i64, vp, i32, i64, vp, i64, i32, vp, vp, vp, vp, vp, vp,
                                   vp, vp]
    L.w4a16_awq_scale.restype = i32
    L.w4a16_awq_scale.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.w4a16_w8a8_smooth.restype = i32
    L.w4a16_w8a8_smooth.argtypes = [vp, i32, i64, vp, i64, i64, i32, vp, vp]
    L.w4a16_w8a8_quantize_weight.restype = i32
    L.w4a16_w8a8_quantize_weight.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.w4a16_w8a8_quantize_act.restype = i32
    L.w4a16_w8a8_quantize_act.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
    L.w4a16_w8a8_linear.restype = i32
    L.w4a16_w8a8_linear.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, i32, vp]
    L.w4a16_kv_attention_workspace.restype = i64
    L.w4a16_kv_attention_workspace.argtypes = [i64, i64, i64]
    L.w4a16_kv_quantize.restype = i32
    L.w4a16_kv_quantize.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp, vp]
    L.w4a16_kv_attention_decode.restype = i32
    L.w4a16_kv_attention_decode.argtypes = [vp, i32, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp]
    L.w4a16_kv_attention_batch_workspace.restype = i64
    L.w4a16_kv_attention_batch_workspace.argtypes = [i64, i64, i64, i64]
    L.w4a16_kv_attention_decode_batch.restype = i32
    L.w4a16_kv_attention_decode_batch.argtypes = [vp, i32, i64, i64, i64, vp, i64, i64, i32, vp, vp, vp, vp,
                                                  vp, vp, vp, vp, vp]
    L.w4a16_gptq_quantize.restype = i32
    L.w4a16_gptq_quantize.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != OK:
        raise W4A16Error(status, what)
