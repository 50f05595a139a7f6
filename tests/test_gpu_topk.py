"""GPU parity tests of the per-row top-k (the top-k form of the decode epilogue): the
kernel's result against the oracle's top-k of the same logits, exactly (indices and values),
on random rows, rows full of ties, special values, strided rows and the lm_head decode."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import TORCH_DTYPE, half_bits, require_gpu

pytestmark = pytest.mark.gpu


def _check(logits, idx, val, k, dtype):
    ref_i, ref_v = O.topk_rows(half_bits(logits), k, dtype)
    got_i = idx.cpu().numpy().astype(np.int64)
    got_v = val.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_i, ref_i), np.argwhere(got_i != ref_i)[:5]
    same = (got_v == ref_v) | (np.isnan(got_v) & np.isnan(ref_v))
    assert same.all()
    # signed zeros are told apart as well (a NaN is reported as a quiet NaN of either sign)
    num = ~np.isnan(ref_v)
    assert np.array_equal(np.signbit(got_v[num]), np.signbit(ref_v[num]))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rows,n,k", [(1, 1, 1), (3, 100, 7), (5, 1000, 64), (2, 4099, 1024), (4, 20000, 50),
                                      (7, 333, 333), (2, 65537, 3), (1, 151936, 50), (1, 151936, 1),
                                      (2, 151936, 200)])
def test_topk_random_rows(rows, n, k, dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    logits = synth.normal_x((rows, n), dtype, seed=1000 + n + k).to(dev)
    for split in (True, False):   # rows over several workgroups, and one workgroup per row
        idx, val = q.topk(logits, k, split=split)
        torch.cuda.synchronize()
        _check(logits, idx, val, k, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("levels,k", [(0, 5), (1, 1), (2, 40), (3, 1024), (50, 200)])
def test_topk_ties(levels, k, dtype):
    # few distinct values: the k-th value is shared by many columns, which must be taken in
    # column order; levels = 0 is an all-equal row
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    logits = synth.tied_logits(6, 3001, levels, dtype, seed=1100 + levels).to(dev)
    idx, val = q.topk(logits, k)
    torch.cuda.synchronize()
    _check(logits, idx, val, k, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_topk_special_values(dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    t = TORCH_DTYPE[dtype]
    base = synth.normal_x((4, 257), dtype, seed=1200).float()
    base[0, [5, 100, 200]] = float("nan")
    base[1, [3, 9]] = float("inf")
    base[1, [4, 10]] = float("-inf")
    base[2, :] = 0.0
    base[2, ::3] = -0.0
    base[3, :] = float("-inf")
    base[3, 250] = float("nan")
    logits = base.to(t).to(dev)
    # NaN payloads and signs other than the canonical quiet NaN count the same
    raw = logits.view(torch.int16)
    raw[0, 100] = torch.tensor(-1, dtype=torch.int16)        # all-ones pattern: a negative NaN
    for k in (1, 4, 257):
        idx, val = q.topk(logits, k)
        torch.cuda.synchronize()
        _check(logits, idx, val, k, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("k", [1, 64, 65])
def test_topk_special_values_long_rows(dtype, k):
    # rows cut into column chunks: NaN (of any payload and sign), infinities and signed zeros
    # inside whole 8-column runs, where the keys are formed two at a time; k = 64 takes the
    # threshold pooled over the waves' largest maxima, k = 65 the least of the waves' values
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    t = TORCH_DTYPE[dtype]
    base = synth.normal_x((3, 20000), dtype, seed=1250).float()
    base[0, [17, 4000, 15001]] = float("nan")
    base[0, [8, 9, 19999]] = float("inf")
    base[1, 100:9000:7] = float("-inf")
    base[1, 5] = -0.0
    base[2, :] = 0.0
    base[2, 1::2] = -0.0
    base[2, [3000, 12000]] = float("nan")
    logits = base.to(t).to(dev)
    raw = logits.view(torch.int16)
    raw[0, 4000] = torch.tensor(-1, dtype=torch.int16)      # a negative NaN
    raw[2, 12000] = torch.tensor(-2, dtype=torch.int16)     # another payload
    ws = q.topk_workspace(3, dev)
    for split in (True, False):
        idx, val = q.topk(logits, k, workspace=ws if split else None, split=split)
        torch.cuda.synchronize()
        _check(logits, idx, val, k, dtype)


def test_topk_strided_rows_and_k1_is_argmax_column():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    wide = synth.tied_logits(9, 900, 4, "bf16", seed=1300).to(dev)
    view = wide[:, 17:17 + 700]                  # row stride 900, 700 columns
    idx, val = q.topk(view, 33)
    torch.cuda.synchronize()
    _check(view.contiguous(), idx, val, 33, "bf16")
    i1, _ = q.topk(view, 1)
    v = view.float().cpu().numpy()
    first_max = [int(np.nonzero(row == row.max())[0][0]) for row in v]
    assert i1[:, 0].cpu().tolist() == first_max


def test_topk_rejects_bad_calls():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    logits = synth.normal_x((2, 10), "bf16", seed=1400).to(dev)
    for k in (0, 11, 1025):
        with pytest.raises(q.QmmError):
            q.topk(logits, k)
    idx, val = q.topk(logits[:0], 3)
    assert idx.shape == (0, 3)


def test_qmv_topk_lm_head():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    c = synth.LM_HEAD
    w = synth.normal_weight(c["n"], c["k"], c["w_std"], seed=c["w_seed"]).to(dev)
    qw = q.quantize(w, c["group_size"], c["bits"], c["dtype"])
    del w
    x = synth.normal_x((c["m"], 1, c["k"]), c["dtype"], seed=c["x_seed"]).to(dev)
    idx, val, y = q.qmv_topk(x, qw, 50)
    y_plain = q.qmv(x, qw)
    am, _, _ = q.qmv_argmax(x, qw, logits=False)
    i1, _, _ = q.qmv_topk(x, qw, 1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))
    assert torch.equal(i1[:, 0], am)
    y2 = y.view(c["m"], c["n"])
    for r in synth.rows_sample(c["m"], 3, seed=1500):
        _check(y2[r:r + 1], idx[r:r + 1], val[r:r + 1], 50, c["dtype"])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("levels,k", [(0, 7), (1, 1000), (2, 1024), (3, 1)])
def test_topk_huge_tie_blocks(levels, k, dtype):
    # more than 4096 keys at or above the threshold bin: the exact-threshold path, whose
    # equal keys are taken in column order across many runs of the row
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    logits = synth.tied_logits(3, 20011, levels, dtype, seed=1600 + levels).to(dev)
    for split in (True, False):
        idx, val = q.topk(logits, k, split=split)
        torch.cuda.synchronize()
        _check(logits, idx, val, k, dtype)


@pytest.mark.parametrize("levels,k", [(2, 120), (40, 300)])
def test_topk_long_rows_large_k(levels, k):
    # chunks longer than the select kernel holds in registers (few chunks per row when k is
    # large): the passes read the chunk from global memory, here with a tie block at the
    # threshold too
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    logits = synth.tied_logits(2, 151936, levels, "bf16", seed=1650 + levels).to(dev)
    for split in (True, False):
        idx, val = q.topk(logits, k, split=split)
        torch.cuda.synchronize()
        _check(logits, idx, val, k, "bf16")


def test_topk_workspace_reuse_and_graph_replay():
    # the workspace needs no initial content (it starts full of 0xA5 bytes here): one
    # workspace serves calls in stream order, eager and replayed from a graph
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    rows, n, k = 5, 50001, 77
    ws = q.topk_workspace(rows, dev)
    ws.view(torch.uint8).fill_(0xA5)
    srcs = [synth.normal_x((rows, n), "bf16", seed=1700 + i).to(dev) for i in range(3)]
    for lg in srcs:
        idx, val = q.topk(lg, k, workspace=ws)
        torch.cuda.synchronize()
        _check(lg, idx, val, k, "bf16")
    buf = srcs[0].clone()
    idx = torch.empty(rows, k, dtype=torch.int32, device=dev)
    val = torch.empty(rows, k, dtype=torch.float32, device=dev)
    q.topk(buf, k, out_index=idx, out_value=val, workspace=ws)   # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.topk(buf, k, out_index=idx, out_value=val, workspace=ws)
    for lg in srcs[::-1]:
        buf.copy_(lg)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(lg, idx, val, k, "bf16")


@pytest.mark.parametrize("dtype,bits,gs", [("fp16", 8, 32), ("bf16", 4, 128), ("fp16", 3, 64)])
def test_qmv_topk_small_and_graph(dtype, bits, gs):
    # decode + top-k on a small weight, eager and replayed from a graph: y equals qmv's, the
    # indices and values equal the oracle's top-k of that y
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, kd, k = 20033, 256, 40
    w = synth.normal_weight(n, kd, 0.02, seed=1800 + bits).to(dev)
    qw = q.quantize(w, gs, bits, dtype)
    x = synth.normal_x((5, 1, kd), dtype, seed=1801).to(dev)
    ws = q.topk_workspace(5, dev)
    idx, val, y = q.qmv_topk(x, qw, k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), q.qmv(x, qw).view(torch.int16))
    _check(y.view(5, n), idx, val, k, dtype)
    yb = torch.empty_like(y)
    ib = torch.empty_like(idx)
    vb = torch.empty_like(val)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qmv_topk(x, qw, k, out=yb, out_index=ib, out_value=vb, workspace=ws)
    for _ in range(3):
        ib.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ib, idx) and torch.equal(vb, val)
