"""Python entry points over the C ABI: quantize, qmv, qmm_t, plan.

Argument marshalling only -- every step of the computation runs in libqmm.so's HIP
kernels.  PyTorch provides device memory and the current HIP stream.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

_DTYPE_CODE = {torch.bfloat16: _lib.QMM_BF16, torch.float16: _lib.QMM_FP16}
_DTYPE_NAME = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass
class QuantizedWeight:
    """Packed codes [N, K*bits/32] (int32 storage of uint32 words), scales/biases [N, K/gs]."""
    w_packed: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    N: int
    K: int
    group_size: int
    bits: int

    @property
    def dtype(self) -> torch.dtype:
        return self.scales.dtype

    def desc(self) -> _lib.WeightDesc:
        d = _lib.WeightDesc()
        d.w_packed = self.w_packed.data_ptr()
        d.w_row_stride = self.w_packed.stride(0)
        d.scales = self.scales.data_ptr()
        d.biases = self.biases.data_ptr()
        assert self.scales.stride() == self.biases.stride() and self.scales.stride(1) == 1
        d.sb_row_stride = self.scales.stride(0)
        d.N, d.K, d.group_size, d.bits = self.N, self.K, self.group_size, self.bits
        d.dtype = _DTYPE_CODE[self.scales.dtype]
        return d


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def quantize(w: torch.Tensor, group_size: int, bits: int, dtype="bf16") -> QuantizedWeight:
    """Quantize a float32 [N, K] device tensor (qmm_quantize)."""
    if isinstance(dtype, str):
        dtype = _DTYPE_NAME[dtype]
    assert w.dtype == torch.float32 and w.dim() == 2 and w.stride(1) == 1 and w.is_cuda
    n, k = w.shape
    lib = _lib.load()
    wp = torch.empty(n, k * bits // 32, dtype=torch.int32, device=w.device)
    sc = torch.empty(n, k // group_size, dtype=dtype, device=w.device)
    bi = torch.empty_like(sc)
    _lib.check(lib.qmm_quantize(w.data_ptr(), n, k, w.stride(0), group_size, bits,
                                _DTYPE_CODE[dtype], wp.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                                _stream(w.device)))
    return QuantizedWeight(wp, sc, bi, n, k, group_size, bits)


def _matmul(entry, x: torch.Tensor, qw: QuantizedWeight, flags: int = 0,
            out: torch.Tensor | None = None) -> torch.Tensor:
    lib = _lib.load()
    y = out if out is not None else torch.empty(*x.shape[:-1], qw.N, dtype=x.dtype, device=x.device)
    xd = _lib.tensor_desc(x.shape, x.stride())
    yd = _lib.tensor_desc(y.shape, y.stride())
    wd = qw.desc()
    if x.dtype != qw.dtype or y.dtype != qw.dtype:
        raise _lib.QmmError(-2, "x, y, scales and biases must share one dtype")
    fn = lib.qmv if entry == 0 else lib.qmm_t
    _lib.check(fn(x.data_ptr(), ctypes.byref(xd), ctypes.byref(wd), y.data_ptr(), ctypes.byref(yd),
                  flags, _stream(x.device)))
    return y


def qmv(x: torch.Tensor, qw: QuantizedWeight, flags: int = 0, out=None) -> torch.Tensor:
    """Decode form, at most 32 collapsed activation rows."""
    return _matmul(0, x, qw, flags, out)


def qmm_t(x: torch.Tensor, qw: QuantizedWeight, flags: int = 0, out=None) -> torch.Tensor:
    """Transposed matrix-matrix form, any number of rows."""
    return _matmul(1, x, qw, flags, out)


@dataclass
class ExpertWeights:
    """A stack of E quantized weights: w_packed [E, N, words], scales/biases [E, N, K/gs]."""
    w_packed: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    N: int
    K: int
    group_size: int
    bits: int

    @staticmethod
    def stack(weights) -> "ExpertWeights":
        q0 = weights[0]
        return ExpertWeights(torch.stack([q.w_packed for q in weights]), torch.stack([q.scales for q in weights]),
                             torch.stack([q.biases for q in weights]), q0.N, q0.K, q0.group_size, q0.bits)

    @property
    def num_experts(self) -> int:
        return self.w_packed.shape[0]

    def expert(self, e: int) -> QuantizedWeight:
        return QuantizedWeight(self.w_packed[e], self.scales[e], self.biases[e], self.N, self.K, self.group_size,
                               self.bits)


def gather_qmv(x: torch.Tensor, experts: ExpertWeights, expert_index: torch.Tensor, out=None) -> torch.Tensor:
    """Row r of x times expert expert_index[r]'s dequantized weight (qmm_gather_qmv)."""
    lib = _lib.load()
    assert expert_index.dtype == torch.int32 and expert_index.is_cuda and expert_index.is_contiguous()
    rows = x.numel() // x.shape[-1] if x.shape[-1] else 0
    if expert_index.numel() != rows:
        raise ValueError("gather_qmv: %d expert indices for %d activation rows" % (expert_index.numel(), rows))
    y = out if out is not None else torch.empty(*x.shape[:-1], experts.N, dtype=x.dtype, device=x.device)
    if x.dtype != experts.scales.dtype or y.dtype != x.dtype:
        raise _lib.QmmError(-2, "x, y, scales and biases must share one dtype")
    wd = experts.expert(0).desc()
    xd = _lib.tensor_desc(x.shape, x.stride())
    yd = _lib.tensor_desc(y.shape, y.stride())
    _lib.check(lib.qmm_gather_qmv(x.data_ptr(), ctypes.byref(xd), ctypes.byref(wd), experts.num_experts,
                                  experts.w_packed.stride(0), experts.scales.stride(0), expert_index.data_ptr(),
                                  y.data_ptr(), ctypes.byref(yd), _stream(x.device)))
    return y


def argmax_workspace(rows: int, device) -> torch.Tensor:
    """A zero-filled workspace for qmv_argmax calls of up to `rows` activation rows; every call
    leaves it zero again, so it can be kept and reused in stream order."""
    return torch.zeros(rows + 1, dtype=torch.int64, device=device)


def qmv_argmax(x: torch.Tensor, qw: QuantizedWeight, logits: bool = True, workspace=None, out=None,
               out_index=None, out_value=None):
    """Decode qmv with a fused per-row argmax (qmm_qmv_argmax).  Returns (index int32 [rows],
    value float32 [rows], y or None); with logits=False the logits are not written.  `out`,
    `out_index` and `out_value` optionally supply the output tensors; `workspace` is one from
    argmax_workspace (a fresh one is allocated when None)."""
    lib = _lib.load()
    rows = x.numel() // x.shape[-1] if x.shape[-1] else 0
    if not logits:
        y = None
    elif out is not None:
        y = out
        assert y.dtype == x.dtype and y.is_contiguous() and tuple(y.shape) == tuple(x.shape[:-1]) + (qw.N,)
    else:
        y = torch.empty(*x.shape[:-1], qw.N, dtype=x.dtype, device=x.device)
    shape = list(x.shape[:-1]) + [qw.N]
    strides, acc = [], 1
    for s in reversed(shape):
        strides.insert(0, acc)
        acc *= s
    yd = _lib.tensor_desc(shape, strides)
    idx = out_index if out_index is not None else torch.empty(rows, dtype=torch.int32, device=x.device)
    val = out_value if out_value is not None else torch.empty(rows, dtype=torch.float32, device=x.device)
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() >= rows
    assert val.dtype == torch.float32 and val.is_contiguous() and val.numel() >= rows
    ws = workspace if workspace is not None else argmax_workspace(rows, x.device)
    assert ws.is_contiguous() and ws.numel() * ws.element_size() >= 8 * (rows + 1)
    if x.dtype != qw.dtype:
        raise _lib.QmmError(-2, "x, scales and biases must share one dtype")
    xd = _lib.tensor_desc(x.shape, x.stride())
    _lib.check(lib.qmm_qmv_argmax(x.data_ptr(), ctypes.byref(xd), ctypes.byref(qw.desc()),
                                  y.data_ptr() if y is not None else None, ctypes.byref(yd), idx.data_ptr(),
                                  val.data_ptr(), ws.data_ptr(), _stream(x.device)))
    return idx, val, y


def qmv_argmax_noalloc(x: torch.Tensor, qw: QuantizedWeight, logits: bool = True, out=None, out_index=None,
                       out_value=None):
    """qmv_argmax without a workspace (qmm_qmv_argmax_noalloc): the library's own device
    array serves as the workspace, so the call allocates nothing when the outputs are given.
    Calls on one GPU that may overlap (different streams) race on that array."""
    lib = _lib.load()
    rows = x.numel() // x.shape[-1] if x.shape[-1] else 0
    if not logits:
        y = None
    elif out is not None:
        y = out
        assert y.dtype == x.dtype and y.is_contiguous() and tuple(y.shape) == tuple(x.shape[:-1]) + (qw.N,)
    else:
        y = torch.empty(*x.shape[:-1], qw.N, dtype=x.dtype, device=x.device)
    shape = list(x.shape[:-1]) + [qw.N]
    strides, acc = [], 1
    for s in reversed(shape):
        strides.insert(0, acc)
        acc *= s
    yd = _lib.tensor_desc(shape, strides)
    idx = out_index if out_index is not None else torch.empty(rows, dtype=torch.int32, device=x.device)
    val = out_value if out_value is not None else torch.empty(rows, dtype=torch.float32, device=x.device)
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() >= rows
    assert val.dtype == torch.float32 and val.is_contiguous() and val.numel() >= rows
    if x.dtype != qw.dtype:
        raise _lib.QmmError(-2, "x, scales and biases must share one dtype")
    xd = _lib.tensor_desc(x.shape, x.stride())
    _lib.check(lib.qmm_qmv_argmax_noalloc(x.data_ptr(), ctypes.byref(xd), ctypes.byref(qw.desc()),
                                          y.data_ptr() if y is not None else None, ctypes.byref(yd), idx.data_ptr(),
                                          val.data_ptr(), _stream(x.device)))
    return idx, val, y


def _dtype_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return _lib.QMM_BF16
    if dtype == torch.float16:
        return _lib.QMM_FP16
    raise _lib.QmmError(-2, "logits must be bfloat16 or float16")


def topk_workspace(rows: int, device) -> torch.Tensor:
    """A workspace for qmm_topk / qmm_qmv_topk over `rows` rows (reusable in stream order;
    its content does not matter)."""
    return torch.empty((32776 * max(rows, 1) + 7) // 8, dtype=torch.int64, device=device)


def topk(logits: torch.Tensor, k: int, out_index=None, out_value=None, workspace=None, split=True):
    """Per-row top-k of a [rows, n] logits tensor (qmm_topk): (index int32 [rows, k], value
    float32 [rows, k]), largest first, equal values by lower column.  With split (default) a
    workspace lets long rows spread over several workgroups (a fresh one is allocated when
    `workspace` is None); split=False runs one workgroup per row."""
    lib = _lib.load()
    assert logits.dim() == 2 and logits.stride(1) == 1
    rows, n = logits.shape
    idx = out_index if out_index is not None else torch.empty(rows, k, dtype=torch.int32, device=logits.device)
    val = out_value if out_value is not None else torch.empty(rows, k, dtype=torch.float32, device=logits.device)
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() >= rows * k
    assert val.dtype == torch.float32 and val.is_contiguous() and val.numel() >= rows * k
    ws = None
    if split:
        ws = workspace if workspace is not None else topk_workspace(rows, logits.device)
        assert ws.is_contiguous() and ws.numel() * ws.element_size() >= 32776 * rows
    _lib.check(lib.qmm_topk(logits.data_ptr(), _dtype_code(logits.dtype), rows, n, logits.stride(0) if rows else n,
                            k, idx.data_ptr(), val.data_ptr(), ws.data_ptr() if ws is not None else None,
                            _stream(logits.device)))
    return idx, val


def qmv_topk(x: torch.Tensor, qw: QuantizedWeight, k: int, out=None, out_index=None, out_value=None,
             workspace=None, split=True):
    """Decode qmv followed by a per-row top-k of its logits (qmm_qmv_topk).  Returns
    (index int32 [rows, k], value float32 [rows, k], y); workspace / split as for topk."""
    lib = _lib.load()
    rows = x.numel() // x.shape[-1] if x.shape[-1] else 0
    if out is not None:
        y = out
        assert y.dtype == x.dtype and y.is_contiguous() and tuple(y.shape) == tuple(x.shape[:-1]) + (qw.N,)
    else:
        y = torch.empty(*x.shape[:-1], qw.N, dtype=x.dtype, device=x.device)
    idx = out_index if out_index is not None else torch.empty(rows, k, dtype=torch.int32, device=x.device)
    val = out_value if out_value is not None else torch.empty(rows, k, dtype=torch.float32, device=x.device)
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.numel() >= rows * k
    assert val.dtype == torch.float32 and val.is_contiguous() and val.numel() >= rows * k
    if x.dtype != qw.dtype:
        raise _lib.QmmError(-2, "x, scales and biases must share one dtype")
    xd = _lib.tensor_desc(x.shape, x.stride())
    yd = _lib.tensor_desc(y.shape, y.stride())
    ws = None
    if split:
        ws = workspace if workspace is not None else topk_workspace(rows, x.device)
        assert ws.is_contiguous() and ws.numel() * ws.element_size() >= 32776 * rows
    _lib.check(lib.qmm_qmv_topk(x.data_ptr(), ctypes.byref(xd), ctypes.byref(qw.desc()), y.data_ptr(),
                                ctypes.byref(yd), k, idx.data_ptr(), val.data_ptr(),
                                ws.data_ptr() if ws is not None else None, _stream(x.device)))
    return idx, val, y


def dequantize(qw: QuantizedWeight, out=None) -> torch.Tensor:
    """Dense [N, K] dtype matrix of the quantized weight (qmm_dequantize)."""
    lib = _lib.load()
    y = out if out is not None else torch.empty(qw.N, qw.K, dtype=qw.dtype, device=qw.w_packed.device)
    assert y.dtype == qw.dtype and y.stride(1) == 1 and tuple(y.shape) == (qw.N, qw.K)
    _lib.check(lib.qmm_dequantize(ctypes.byref(qw.desc()), y.data_ptr(), y.stride(0), _stream(y.device)))
    return y


def embedding(qw: QuantizedWeight, indices: torch.Tensor, out=None) -> torch.Tensor:
    """Dequantized rows indices[r] of a quantized table (qmm_embedding); NaN rows for indices
    outside [0, N)."""
    lib = _lib.load()
    assert indices.dtype == torch.int32 and indices.is_cuda and indices.is_contiguous()
    count = indices.numel()
    y = out if out is not None else torch.empty(count, qw.K, dtype=qw.dtype, device=indices.device)
    assert y.dtype == qw.dtype and y.stride(1) == 1 and tuple(y.shape) == (count, qw.K)
    _lib.check(lib.qmm_embedding(ctypes.byref(qw.desc()), indices.data_ptr(), count, y.data_ptr(), y.stride(0),
                                 _stream(y.device)))
    return y


def plan(x_shape, x_stride, N: int, K: int, group_size: int = 64, bits: int = 4,
         dtype: int = _lib.QMM_BF16, entry: int = 1, flags: int = 0, y_shape=None, y_stride=None,
         w_row_stride=None) -> dict:
    """Host-only dispatcher query (qmm_plan): the plan, or QmmError.  The weight row stride
    defaults to the packed row padded to a multiple of 4 words."""
    lib = _lib.load()
    if y_shape is None:
        y_shape = list(x_shape[:-1]) + [N]
    if y_stride is None:
        y_stride, acc = [], 1
        for s in reversed(y_shape):
            y_stride.insert(0, acc)
            acc *= s
    xd = _lib.tensor_desc(x_shape, x_stride)
    yd = _lib.tensor_desc(y_shape, y_stride)
    wd = _lib.WeightDesc()
    wd.w_row_stride = K * bits // 32 + (-(K * bits // 32)) % 4 if w_row_stride is None else w_row_stride
    wd.sb_row_stride = K // group_size
    wd.N, wd.K, wd.group_size, wd.bits, wd.dtype = N, K, group_size, bits, dtype
    p = _lib.Plan()
    _lib.check(lib.qmm_plan(ctypes.byref(xd), ctypes.byref(wd), ctypes.byref(yd), flags, entry,
                            ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in _lib.Plan._fields_}
