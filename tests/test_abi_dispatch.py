"""CPU tests of the boundary: the library loads and exports every declared symbol, and the
host dispatcher (qmm_plan, no GPU) folds or rejects layouts as specified."""
import ctypes
import os
import re

import pytest

import bit_affine_quantized_qmv_amd as q
from bit_affine_quantized_qmv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qmm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = q.load()
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name
    assert lib.qmm_abi_version() == 1
    assert lib.qmm_last_error() == b""


def _plan(shape, stride, **kw):
    return q.plan(shape, stride, kw.pop("N", 64), shape[-1], **kw)


def _dense(shape):
    st, acc = [], 1
    for s in reversed(shape):
        st.insert(0, acc)
        acc *= s
    return st


def _err(shape, stride, code, **kw):
    with pytest.raises(q.QmmError) as e:
        _plan(shape, stride, **kw)
    assert e.value.code == code, e.value
    return e.value.message


K = 1024


def test_two_d_and_vector():
    p = _plan([7, K], [K, 1])
    assert (p["rows"], p["kind"], p["family"], p["seg_rows"], p["row_stride"]) == (7, 0, 0, 7, K)
    p = _plan([K], [1])
    assert (p["rows"], p["kind"], p["family"]) == (1, 0, 0)


def test_batched_decode_folds_to_2d():
    """[B,1,K] folds to M=B rows at the batch stride (transformers issue 47331, Fix)."""
    for b in (1, 2, 4, 8, 16, 32):
        p = _plan([b, 1, K], [K, K, 1])
        assert (p["rows"], p["kind"], p["batches"]) == (b, 0, 1)
        assert p["row_stride"] == (K if b > 1 else p["row_stride"])
    p = _plan([16, 1, K], [2 * K, K, 1])          # evenly strided rows
    assert (p["rows"], p["kind"], p["row_stride"]) == (16, 0, 2 * K)
    p = _plan([2, 4, K], [4 * K, K, 1])
    assert (p["rows"], p["kind"], p["row_stride"]) == (8, 0, K)


def test_forced_strided_splits_batches():
    p = _plan([32, 1, K], [K, K, 1], flags=q.QMM_FLAG_FORCE_STRIDED)
    assert (p["kind"], p["batches"], p["batch_stride"], p["rows_per_batch"], p["family"]) == \
        (2, 32, K, 1, 0)
    p = _plan([4, 512, 4096], [1024 * 4096, 4096, 1], N=14336, group_size=128,
              flags=q.QMM_FLAG_FORCE_STRIDED)
    assert (p["kind"], p["batches"], p["rows_per_batch"], p["family"]) == (2, 4, 512, 1)


def test_prefill_view_two_levels():
    p = _plan([4, 512, 4096], [1024 * 4096, 4096, 1], N=14336, group_size=128)
    assert (p["rows"], p["kind"], p["family"], p["seg_rows"], p["seg_stride"], p["row_stride"]) == \
        (2048, 1, 1, 512, 1024 * 4096, 4096)
    p = _plan([4, 512, 4096], [512 * 4096, 4096, 1], N=14336, group_size=128)
    assert (p["rows"], p["kind"], p["family"]) == (2048, 0, 1)


def test_candle_layouts_fold_into_two_levels():
    """candle pitfall page: (2,4,5,d) at strides (480,40,8,1)-shaped, (2,2,3,d) at (60,15,5,1)-
    shaped, and a rank-5 contiguous input (which candle's CPU path wrongly rejects)."""
    d = 128
    p = _plan([2, 4, 5, d], [12 * 5 * d, 5 * d, d, 1])
    assert (p["rows"], p["kind"], p["seg_rows"], p["row_stride"], p["seg_stride"]) == \
        (40, 1, 20, d, 60 * d)
    p = _plan([2, 2, 3, d], [4 * 3 * d, 3 * d, d, 1])
    assert (p["rows"], p["kind"], p["seg_rows"]) == (12, 1, 6)
    p = _plan([2, 2, 2, 3, d], _dense([2, 2, 2, 3, d]))
    assert (p["rows"], p["kind"], p["row_stride"]) == (24, 0, d)


def test_broadcast_rows():
    p = _plan([4, 3, K], [K, 0, 1])
    assert (p["rows"], p["kind"], p["seg_rows"], p["row_stride"], p["seg_stride"]) == (12, 1, 3, 0, K)
    p = _plan([5, K], [0, 1])
    assert (p["rows"], p["kind"], p["row_stride"]) == (5, 0, 0)


def test_three_levels_rejected_with_layout_in_message():
    msg = _err([2, 2, 3, 4, 128], [5 * 4 * 3 * 128 * 2, 4 * 5 * 128, 5 * 128, 128, 1], -4, group_size=32)
    assert "shape [2, 2, 3, 4, 128]" in msg and "stride [" in msg


def test_rejections():
    _err([3, K], [K, 2], -4)                       # last-dim stride != 1
    _err([3, K], [-K, 1], -4)                      # negative stride
    _err([3, 96], [96, 1], -3, group_size=64)      # K not a multiple of group_size
    _err([3, K], [K, 1], -2, bits=7)
    _err([3, K], [K, 1], -2, group_size=16)
    _err([3, K], [K, 1], -2, dtype=3)
    _err([33, K], [K, 1], -3, entry=0)             # qmv takes at most 32 rows
    _err([3, K], [K, 1], -3, y_shape=[3, 63])
    _err([3, K], [K, 1], -4, y_shape=[3, 64], y_stride=[128, 1])
    _err([3, K], [K + 4, 1], -5)                   # row stride not a multiple of 8 elements
    _err([3, K], [K, 1], -2, flags=1 << 5)


def test_empty_is_a_plan():
    p = _plan([0, K], [K, 1])
    assert p["rows"] == 0
    p = _plan([0, 5, K], [5 * K, K, 1], entry=0)
    assert p["rows"] == 0
    p = _plan([3, K], [K, 1], N=0)
    assert p["rows"] == 3


def test_unaligned_k_and_odd_row_strides():
    """K a multiple of the group size but not of 128 stays on the decode kernels up to 32
    rows (their last slot is masked); weight rows padded to a word count the decode kernels
    cannot load in 16-byte pieces plan the MFMA kernel at every row count (MLX pull request
    4516, second commit text: unaligned inputs take the generic kernel)."""
    for m in (1, 7, 32, 33, 500):
        dec = 0 if m <= 32 else 1
        p = _plan([m, 1056], [1056, 1], group_size=32)
        assert (p["rows"], p["family"]) == (m, dec)
        p = _plan([m, 1088], [1088, 1], group_size=64, entry=0 if m <= 32 else 1)
        assert p["family"] == dec
        assert _plan([m, K], [K, 1], bits=3, w_row_stride=97)["family"] == 1
        assert _plan([m, K], [K, 1], bits=3, w_row_stride=100)["family"] == dec
    assert _plan([4, 32], [32, 1], group_size=32, entry=0)["family"] == 0
    # the run alignment of each code width: 4 words for 4/8-bit, 2 for 2/6-bit, 1 otherwise
    _err([3, K], [K, 1], -5, bits=4, w_row_stride=130)
    _err([3, K], [K, 1], -5, bits=8, w_row_stride=258)
    _err([3, K], [K, 1], -5, bits=6, w_row_stride=193)
    _err([3, K], [K, 1], -5, bits=2, w_row_stride=65)
    assert _plan([3, K], [K, 1], bits=6, w_row_stride=194)["family"] == 1
    assert _plan([3, K], [K, 1], bits=5, w_row_stride=161)["family"] == 1
    _err([3, K], [K, 1], -3, bits=5, w_row_stride=159)   # shorter than a row


def test_qmv_family_boundary():
    assert _plan([32, K], [K, 1], entry=0)["family"] == 0
    assert _plan([33, K], [K, 1])["family"] == 1
    assert _plan([32, 1, K], [K, K, 1])["family"] == 0


def test_error_message_is_thread_local_and_cleared():
    lib = q.load()
    with pytest.raises(q.QmmError):
        _plan([3, K], [K, 2])
    assert lib.qmm_last_error() != b""
    _plan([3, K], [K, 1])
    assert lib.qmm_last_error() == b""


def test_topk_validation_before_any_launch():
    # every rejection happens on the host, before anything is enqueued (no GPU needed)
    lib = q.load()
    codes = {name: code for code, name in _lib.ERRORS.items()}
    assert lib.qmm_topk(None, 1, 4, 10, 10, 0, None, None, None, None) == codes["QMM_ERR_SHAPE"]
    assert lib.qmm_topk(None, 1, 4, 10, 10, 11, None, None, None, None) == codes["QMM_ERR_SHAPE"]
    assert lib.qmm_topk(None, 1, 4, 2000, 2000, 1025, None, None, None, None) == codes["QMM_ERR_SHAPE"]
    assert lib.qmm_topk(None, 1, 4, 10, 9, 3, None, None, None, None) == codes["QMM_ERR_SHAPE"]
    assert lib.qmm_topk(None, 1, -1, 10, 10, 3, None, None, None, None) == codes["QMM_ERR_SHAPE"]
    assert lib.qmm_topk(None, 3, 4, 10, 10, 3, None, None, None, None) == codes["QMM_ERR_UNSUPPORTED"]
    assert b"dtype" in lib.qmm_last_error()
    assert lib.qmm_topk(None, 1, 4, 10, 10, 3, None, None, None, None) == codes["QMM_ERR_NULL"]
    assert lib.qmm_topk(None, 2, 0, 10, 10, 3, None, None, None, None) == 0   # no rows: a no-op
    assert lib.qmm_last_error() == b""
