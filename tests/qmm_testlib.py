"""Helpers shared by the GPU parity tests: move data between torch and the oracle.

Test infrastructure: converts tensors to the bit patterns / float64 values the oracle
takes; no quantization or matmul arithmetic happens here.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_affine_quantized_qmv_amd as q
    q.load()  # fail loudly if the library is missing
    return torch.device("cuda:0")


def half_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16/fp16 tensor (copied to host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def values(t: torch.Tensor) -> np.ndarray:
    """float64 values of a bf16/fp16/fp32 tensor (exact)."""
    return t.detach().cpu().float().numpy().astype(np.float64)


def words(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def upload_oracle_weight(q_oracle: dict, device) -> "object":
    """Hand an oracle-quantized weight (codes packed by the oracle) to the library."""
    import bit_affine_quantized_qmv_amd as q
    bits, gs, dt = q_oracle["bits"], q_oracle["group_size"], q_oracle["dtype"]
    packed = O.pack(q_oracle["codes"], bits)
    n, k = q_oracle["codes"].shape
    wp = torch.from_numpy(packed.view(np.int32).copy()).to(device)
    sc = torch.from_numpy(q_oracle["scales_bits"].view(np.int16).copy()).view(TORCH_DTYPE[dt]).to(device)
    bi = torch.from_numpy(q_oracle["biases_bits"].view(np.int16).copy()).view(TORCH_DTYPE[dt]).to(device)
    return q.QuantizedWeight(wp, sc, bi, n, k, gs, bits)


def oracle_view_of(qw) -> dict:
    """The library's weight triple copied back as oracle inputs (words, scale/bias bits)."""
    return {"w_packed": words(qw.w_packed), "scales_bits": half_bits(qw.scales),
            "biases_bits": half_bits(qw.biases)}


def reference_rows(x_rows: np.ndarray, qw, dtype: str, rows=None) -> dict:
    """y_ref and tolerance for float64 activation rows against the weight in `qw`."""
    ov = oracle_view_of(qw)
    return O.reference(x_rows, ov["w_packed"], ov["scales_bits"], ov["biases_bits"], qw.K,
                       qw.group_size, qw.bits, dtype, rows=rows)


def gather(buf: torch.Tensor, view: torch.Tensor) -> np.ndarray:
    """Activation rows of `view` (a view into `buf`) gathered by the oracle from buf's
    flat storage using the view's shape, strides and offset."""
    flat = values(buf.reshape(-1))
    off = view.storage_offset() - buf.storage_offset()
    return O.gather_rows(flat, list(view.shape), list(view.stride()), off)


def assert_close(y: torch.Tensor, ref: dict, what: str = ""):
    yv = values(y).reshape(ref["y_ref"].shape)
    res = O.check(yv, ref["y_ref"], ref["tol"])
    assert res["ok"], "%s: %d elements outside the bound, worst ratio %.3g, first %s" % (
        what, res["n_bad"], res["worst_ratio"], res["first_bad"])
    return res
