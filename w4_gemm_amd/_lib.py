"""ctypes binding of libsq (include/sq.h).  Argument marshalling only.

The library must have been built (``python -m w4_gemm_amd.build``); there is
no fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsq.so")

SQ_OK = 0
SQ_F32, SQ_BF16 = 0, 1
SQ_FLAG_NONFINITE, SQ_FLAG_SCALE_OVERFLOW, SQ_FLAG_FP16_RANGE = 1, 2, 4
STATUS_NAMES = {0: "SQ_OK", 1: "SQ_E_NULL", 2: "SQ_E_SHAPE", 3: "SQ_E_GROUP", 4: "SQ_E_RANK",
                5: "SQ_E_ALIGN", 6: "SQ_E_WORKSPACE", 7: "SQ_E_DTYPE", 8: "SQ_E_ARCH",
                9: "SQ_E_HIP"}

# every symbol include/sq.h declares
EXPORTS = ("sq_quantize_weight", "sq_linear_fwd_workspace_bytes", "sq_linear_fwd",
           "sq_linear_fwd_rotate", "sq_linear_fwd_contract", "sq_reconstruct_bf16",
           "sq_linear_dgrad_workspace_bytes", "sq_linear_dgrad", "sq_status_str",
           "sq_abi_version", "sq_quantize_weight_w8_workspace_bytes", "sq_quantize_weight_w8",
           "sq_reconstruct_bf16_w8", "sq_linear_fwd_w8_workspace_bytes", "sq_linear_fwd_w8",
           "sq_quantize_weight_mx4", "sq_quantize_act_mx4", "sq_reconstruct_bf16_mx4",
           "sq_linear_fwd_mx4_workspace_bytes", "sq_linear_fwd_mx4", "sq_linear_fwd_static")
SQ_FWD_STATIC_SCRATCH_BYTES = 64 << 20


class SqW4(ctypes.Structure):
    """Mirror of sq_w4_t."""
    _fields_ = [
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("group", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("lora_up", ctypes.c_void_p),
        ("lora_down", ctypes.c_void_p),
    ]


class SqW8(ctypes.Structure):
    """Mirror of sq_w8_t (int8-residual mode)."""
    _fields_ = [
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("rank", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("lora_up", ctypes.c_void_p),
        ("lora_down", ctypes.c_void_p),
    ]


class SqMx4(ctypes.Structure):
    """Mirror of sq_mx4_t (MXFP4 mode)."""
    _fields_ = [
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("rank", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("exps", ctypes.c_void_p),
        ("lora_up", ctypes.c_void_p),
        ("lora_down", ctypes.c_void_p),
    ]


class SqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.sq_quantize_weight.argtypes = [vp, ctypes.POINTER(SqW4), vp, vp, vp]
        L.sq_quantize_weight.restype = ctypes.c_int
        L.sq_linear_fwd_workspace_bytes.argtypes = [i64, ctypes.POINTER(SqW4)]
        L.sq_linear_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.sq_linear_fwd.argtypes = [vp, i64, ctypes.POINTER(SqW4), vp, ctypes.c_int, vp,
                                    ctypes.c_size_t, vp]
        L.sq_linear_fwd.restype = ctypes.c_int
        L.sq_linear_fwd_rotate.argtypes = [vp, i64, ctypes.POINTER(SqW4), vp, ctypes.c_size_t, vp]
        L.sq_linear_fwd_rotate.restype = ctypes.c_int
        L.sq_linear_fwd_contract.argtypes = [i64, ctypes.POINTER(SqW4), vp, ctypes.c_int, vp,
                                             ctypes.c_size_t, vp]
        L.sq_linear_fwd_contract.restype = ctypes.c_int
        L.sq_linear_dgrad_workspace_bytes.argtypes = [i64, ctypes.POINTER(SqW4)]
        L.sq_linear_dgrad_workspace_bytes.restype = ctypes.c_size_t
        L.sq_linear_dgrad.argtypes = [vp, i64, ctypes.POINTER(SqW4), vp, ctypes.c_int, vp,
                                      ctypes.c_size_t, vp]
        L.sq_linear_dgrad.restype = ctypes.c_int
        L.sq_linear_fwd_static.argtypes = [vp, i64, ctypes.POINTER(SqW4), vp, ctypes.c_int, vp]
        L.sq_linear_fwd_static.restype = ctypes.c_int
        L.sq_reconstruct_bf16.argtypes = [ctypes.POINTER(SqW4), vp, vp]
        L.sq_reconstruct_bf16.restype = ctypes.c_int
        P8 = ctypes.POINTER(SqW8)
        L.sq_quantize_weight_w8_workspace_bytes.argtypes = [P8]
        L.sq_quantize_weight_w8_workspace_bytes.restype = ctypes.c_size_t
        L.sq_quantize_weight_w8.argtypes = [vp, P8, vp, vp, vp, ctypes.c_size_t, vp]
        L.sq_quantize_weight_w8.restype = ctypes.c_int
        L.sq_reconstruct_bf16_w8.argtypes = [P8, vp, vp]
        L.sq_reconstruct_bf16_w8.restype = ctypes.c_int
        L.sq_linear_fwd_w8_workspace_bytes.argtypes = [i64, P8]
        L.sq_linear_fwd_w8_workspace_bytes.restype = ctypes.c_size_t
        L.sq_linear_fwd_w8.argtypes = [vp, i64, P8, vp, ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.sq_linear_fwd_w8.restype = ctypes.c_int
        PX = ctypes.POINTER(SqMx4)
        L.sq_quantize_weight_mx4.argtypes = [vp, PX, vp, vp]
        L.sq_quantize_weight_mx4.restype = ctypes.c_int
        L.sq_quantize_act_mx4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.sq_quantize_act_mx4.restype = ctypes.c_int
        L.sq_reconstruct_bf16_mx4.argtypes = [PX, vp, vp]
        L.sq_reconstruct_bf16_mx4.restype = ctypes.c_int
        L.sq_linear_fwd_mx4_workspace_bytes.argtypes = [i64, PX]
        L.sq_linear_fwd_mx4_workspace_bytes.restype = ctypes.c_size_t
        L.sq_linear_fwd_mx4.argtypes = [vp, i64, PX, vp, ctypes.c_int, vp, ctypes.c_size_t, vp]
        L.sq_linear_fwd_mx4.restype = ctypes.c_int
        L.sq_status_str.argtypes = [ctypes.c_int]
        L.sq_status_str.restype = ctypes.c_char_p
        L.sq_abi_version.argtypes = []
        L.sq_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().sq_status_str(status).decode()


def abi_version() -> int:
    return lib().sq_abi_version()


def sq_quantize_weight(w, p: SqW4, fidx, dev_flags, stream) -> int:
    return lib().sq_quantize_weight(w, ctypes.byref(p), fidx, dev_flags, stream)


def sq_linear_fwd_workspace_bytes(m: int, p: SqW4) -> int:
    return lib().sq_linear_fwd_workspace_bytes(m, ctypes.byref(p))


def sq_linear_fwd(x, m: int, p: SqW4, y, y_dtype: int, workspace, workspace_bytes: int,
                  stream) -> int:
    return lib().sq_linear_fwd(x, m, ctypes.byref(p), y, y_dtype, workspace, workspace_bytes,
                               stream)


def sq_linear_fwd_rotate(x, m: int, p: SqW4, workspace, workspace_bytes: int, stream) -> int:
    return lib().sq_linear_fwd_rotate(x, m, ctypes.byref(p), workspace, workspace_bytes, stream)


def sq_linear_fwd_contract(m: int, p: SqW4, y, y_dtype: int, workspace, workspace_bytes: int,
                           stream) -> int:
    return lib().sq_linear_fwd_contract(m, ctypes.byref(p), y, y_dtype, workspace,
                                        workspace_bytes, stream)


def sq_linear_fwd_static(x, m: int, p: SqW4, y, y_dtype: int, stream) -> int:
    return lib().sq_linear_fwd_static(x, m, ctypes.byref(p), y, y_dtype, stream)


def sq_reconstruct_bf16(p: SqW4, w_hat, stream) -> int:
    return lib().sq_reconstruct_bf16(ctypes.byref(p), w_hat, stream)


def sq_linear_dgrad_workspace_bytes(m: int, p: SqW4) -> int:
    return lib().sq_linear_dgrad_workspace_bytes(m, ctypes.byref(p))


def sq_linear_dgrad(dy, m: int, p: SqW4, dx, dx_dtype: int, workspace, workspace_bytes: int,
                    stream) -> int:
    return lib().sq_linear_dgrad(dy, m, ctypes.byref(p), dx, dx_dtype, workspace,
                                 workspace_bytes, stream)


def sq_quantize_weight_w8_workspace_bytes(p: SqW8) -> int:
    return lib().sq_quantize_weight_w8_workspace_bytes(ctypes.byref(p))


def sq_quantize_weight_w8(w, p: SqW8, fidx, dev_flags, workspace, workspace_bytes: int,
                          stream) -> int:
    return lib().sq_quantize_weight_w8(w, ctypes.byref(p), fidx, dev_flags, workspace,
                                       workspace_bytes, stream)


def sq_reconstruct_bf16_w8(p: SqW8, w_hat, stream) -> int:
    return lib().sq_reconstruct_bf16_w8(ctypes.byref(p), w_hat, stream)


def sq_linear_fwd_w8_workspace_bytes(m: int, p: SqW8) -> int:
    return lib().sq_linear_fwd_w8_workspace_bytes(m, ctypes.byref(p))


def sq_linear_fwd_w8(x, m: int, p: SqW8, y, y_dtype: int, workspace, workspace_bytes: int,
                     stream) -> int:
    return lib().sq_linear_fwd_w8(x, m, ctypes.byref(p), y, y_dtype, workspace, workspace_bytes,
                                  stream)


def sq_quantize_weight_mx4(w, p: SqMx4, dev_flags, stream) -> int:
    return lib().sq_quantize_weight_mx4(w, ctypes.byref(p), dev_flags, stream)


def sq_quantize_act_mx4(x, m: int, k: int, xq, xs, stream) -> int:
    return lib().sq_quantize_act_mx4(x, m, k, xq, xs, stream)


def sq_reconstruct_bf16_mx4(p: SqMx4, w_hat, stream) -> int:
    return lib().sq_reconstruct_bf16_mx4(ctypes.byref(p), w_hat, stream)


def sq_linear_fwd_mx4_workspace_bytes(m: int, p: SqMx4) -> int:
    return lib().sq_linear_fwd_mx4_workspace_bytes(m, ctypes.byref(p))


def sq_linear_fwd_mx4(x, m: int, p: SqMx4, y, y_dtype: int, workspace, workspace_bytes: int,
                      stream) -> int:
    return lib().sq_linear_fwd_mx4(x, m, ctypes.byref(p), y, y_dtype, workspace, workspace_bytes,
                                   stream)
