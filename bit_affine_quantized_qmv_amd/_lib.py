"""ctypes declarations of libqmm.so (the C ABI in include/qmm.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os

QMM_MAX_DIMS = 8
QMM_DECODE_MAX_ROWS = 32
QMM_BF16 = 1
QMM_FP16 = 2
QMM_FLAG_FORCE_STRIDED = 1

ERRORS = {
    0: "QMM_OK",
    -1: "QMM_ERR_NULL",
    -2: "QMM_ERR_UNSUPPORTED",
    -3: "QMM_ERR_SHAPE",
    -4: "QMM_ERR_LAYOUT",
    -5: "QMM_ERR_ALIGN",
    -6: "QMM_ERR_HIP",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmm.so")

# Every symbol include/qmm.h declares.
EXPORTS = ("qmm_abi_version", "qmm_last_error", "qmm_quantize", "qmv", "qmm_t", "qmm_plan", "qmm_gather_qmv",
           "qmm_dequantize", "qmm_embedding", "qmm_qmv_argmax", "qmm_qmv_argmax_noalloc", "qmm_topk",
           "qmm_qmv_topk")


class TensorDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * QMM_MAX_DIMS),
                ("stride", ctypes.c_int64 * QMM_MAX_DIMS)]


class WeightDesc(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p),
                ("w_row_stride", ctypes.c_int64),
                ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p),
                ("sb_row_stride", ctypes.c_int64),
                ("N", ctypes.c_int64),
                ("K", ctypes.c_int64),
                ("group_size", ctypes.c_int32),
                ("bits", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64),
                ("batches", ctypes.c_int64),
                ("batch_stride", ctypes.c_int64),
                ("rows_per_batch", ctypes.c_int64),
                ("seg_rows", ctypes.c_int64),
                ("seg_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64),
                ("family", ctypes.c_int32),
                ("kind", ctypes.c_int32)]


class QmmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, message))
        self.code = code
        self.message = message


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libqmm.so; fail loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqmm.so is not built (%s); run `python -m bit_affine_quantized_qmv_amd.build`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.qmm_abi_version.restype = ctypes.c_int32
    lib.qmm_abi_version.argtypes = []
    lib.qmm_last_error.restype = ctypes.c_char_p
    lib.qmm_last_error.argtypes = []
    lib.qmm_quantize.restype = ctypes.c_int32
    lib.qmm_quantize.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    for name in ("qmv", "qmm_t"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int32
        fn.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc), P,
                       ctypes.POINTER(TensorDesc), ctypes.c_uint32, P]
    lib.qmm_gather_qmv.restype = ctypes.c_int32
    lib.qmm_gather_qmv.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc), ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, P, P, ctypes.POINTER(TensorDesc), P]
    lib.qmm_qmv_argmax.restype = ctypes.c_int32
    lib.qmm_qmv_argmax.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc), P,
                                   ctypes.POINTER(TensorDesc), P, P, P, P]
    lib.qmm_qmv_argmax_noalloc.restype = ctypes.c_int32
    lib.qmm_qmv_argmax_noalloc.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc), P,
                                           ctypes.POINTER(TensorDesc), P, P, P]
    lib.qmm_topk.restype = ctypes.c_int32
    lib.qmm_topk.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                             P, P, P, P]
    lib.qmm_qmv_topk.restype = ctypes.c_int32
    lib.qmm_qmv_topk.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc), P,
                                 ctypes.POINTER(TensorDesc), ctypes.c_int32, P, P, P, P]
    lib.qmm_dequantize.restype = ctypes.c_int32
    lib.qmm_dequantize.argtypes = [ctypes.POINTER(WeightDesc), P, ctypes.c_int64, P]
    lib.qmm_embedding.restype = ctypes.c_int32
    lib.qmm_embedding.argtypes = [ctypes.POINTER(WeightDesc), P, ctypes.c_int64, P, ctypes.c_int64, P]
    lib.qmm_plan.restype = ctypes.c_int32
    lib.qmm_plan.argtypes = [ctypes.POINTER(TensorDesc), ctypes.POINTER(WeightDesc),
                             ctypes.POINTER(TensorDesc), ctypes.c_uint32, ctypes.c_int32,
                             ctypes.POINTER(Plan)]
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != 0:
        raise QmmError(rc, load().qmm_last_error().decode())


def tensor_desc(shape, stride) -> TensorDesc:
    d = TensorDesc()
    d.ndim = len(shape)
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = int(s)
        d.stride[i] = int(st)
    return d
