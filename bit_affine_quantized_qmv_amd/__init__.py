"""Affine group-quantized matmul (qmv / qmm_t) on AMD MI355X (gfx950).

The computation lives in libqmm.so (hand-written HIP kernels behind the C ABI of
include/qmm.h); this package only marshals torch tensors into those calls.
"""
from ._lib import (QMM_BF16, QMM_DECODE_MAX_ROWS, QMM_FLAG_FORCE_STRIDED, QMM_FP16, QmmError,
                   load)
from .api import (ExpertWeights, QuantizedWeight, argmax_workspace, dequantize, embedding, gather_qmv, plan, qmm_t, qmv,
                  qmv_argmax, qmv_argmax_noalloc, qmv_topk, quantize, topk, topk_workspace)

__all__ = ["QMM_BF16", "QMM_FP16", "QMM_FLAG_FORCE_STRIDED", "QMM_DECODE_MAX_ROWS", "QmmError",
           "QuantizedWeight", "ExpertWeights", "argmax_workspace", "dequantize", "embedding", "gather_qmv", "qmv_argmax", "qmv_argmax_noalloc", "qmv_topk", "topk", "topk_workspace", "load", "plan", "qmm_t", "qmv", "quantize"]
