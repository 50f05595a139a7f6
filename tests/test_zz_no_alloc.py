"""The decode + argmax entry point that allocates nothing (qmm_qmv_argmax_noalloc), against
the one that takes a caller workspace (qmm_qmv_argmax): bitwise the same index, value and
logits, on consecutive calls of different sizes (the library's scratch keeps the previous
call's contents), without logits, and replayed from a captured graph."""
import pytest
import torch

import synth
from qmm_testlib import require_gpu

pytestmark = pytest.mark.gpu


def _pair(q, dev, m, n, k, bits, gs, dtype, seed):
    qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=seed).to(dev), gs, bits, dtype)
    x = synth.normal_x((m, 1, k), dtype, seed=seed + 1).to(dev)
    return qw, x


def test_noalloc_argmax_equals_workspace_argmax_on_consecutive_calls():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    # second call smaller: fewer rows, another width, another kernel
    for m, n, k, bits, gs, dtype in ((32, 3001, 1024, 4, 64, "bf16"), (5, 777, 512, 8, 32, "fp16")):
        qw, x = _pair(q, dev, m, n, k, bits, gs, dtype, seed=m + n)
        ws = q.argmax_workspace(m, dev)
        i0, v0, y0 = q.qmv_argmax(x, qw, workspace=ws)
        i1, v1, y1 = q.qmv_argmax_noalloc(x, qw)
        torch.cuda.synchronize()
        assert torch.equal(i1, i0) and torch.equal(v1, v0) and torch.equal(y1, y0), (m, n, bits)
        assert torch.equal(i1.long(), y1.float().reshape(m, n).argmax(dim=1)), (m, n)
        i2, v2, y2 = q.qmv_argmax_noalloc(x, qw, logits=False)
        assert y2 is None and torch.equal(i2, i0) and torch.equal(v2, v0), (m, n, bits)


def test_noalloc_argmax_graph_replays():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    qw, x = _pair(q, dev, 16, 2000, 1024, 4, 64, "bf16", seed=7)
    ws = q.argmax_workspace(16, dev)
    i0, v0, y0 = q.qmv_argmax(x, qw, workspace=ws)
    idx = torch.empty(16, dtype=torch.int32, device=dev)
    val = torch.empty(16, dtype=torch.float32, device=dev)
    y = torch.empty_like(y0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qmv_argmax_noalloc(x, qw, out=y, out_index=idx, out_value=val)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qmv_argmax_noalloc(x, qw, out=y, out_index=idx, out_value=val)
    for r in range(4):
        idx.fill_(-1)
        val.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, i0) and torch.equal(val, v0) and torch.equal(y, y0), r
        # eager work of the program between replays
        i3, v3, _ = q.qmv_argmax_noalloc(x[:3], qw, logits=False)
        torch.cuda.synchronize()
        assert torch.equal(i3, i0[:3]), r
