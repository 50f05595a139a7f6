"""GPU parity tests of the rows that extend the hot path: gathered-weight decode, ..."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import TORCH_DTYPE, assert_close, half_bits, require_gpu, upload_oracle_weight, values, words

pytestmark = pytest.mark.gpu


def _experts(n, k, gs, bits, dtype, count, seed, dev):
    import bit_affine_quantized_qmv_amd as q
    ws = []
    for e in range(count):
        w = synth.normal_weight(n, k, 0.02, seed=seed + e).numpy()
        ws.append(upload_oracle_weight(O.quantize(w, gs, bits, dtype), dev))
    return q.ExpertWeights.stack(ws), ws


def _oracle_triples(ws):
    return [(words(q.w_packed), half_bits(q.scales), half_bits(q.biases)) for q in ws]


@pytest.mark.parametrize("bits,gs,dtype", [(4, 64, "bf16"), (8, 64, "fp16"), (3, 32, "bf16"), (4, 128, "fp16")])
def test_gather_qmv_parity(bits, gs, dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k, e = 1000, 1024, 5
    ex, ws = _experts(n, k, gs, bits, dtype, e, 700, dev)
    idx = torch.tensor([3, 0, 4, 4, 1, 3, 2], dtype=torch.int32, device=dev)
    x = synth.normal_x((7, k), dtype, seed=71).to(dev)
    y = q.gather_qmv(x, ex, idx)
    torch.cuda.synchronize()
    ref = O.gather_reference(values(x), _oracle_triples(ws), idx.cpu().numpy(), k, gs, bits, dtype)
    assert_close(y, ref, "gather_qmv")
    # each row is the plain decode call on that row with its expert, bit for bit
    for r in range(7):
        y1 = q.qmv(x[r:r + 1], ws[int(idx[r])])
        assert torch.equal(y1[0].view(torch.int16), y[r].view(torch.int16)), r


def test_gather_qmv_bad_index_rows_nan_and_padded_stride():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k, gs, bits, dtype = 333, 512, 64, 4, "bf16"
    ex, ws = _experts(n, k, gs, bits, dtype, 3, 720, dev)
    # expert stack with padded per-expert strides (extra rows of NaN-poisoned scales)
    words_pad = torch.zeros(3, n + 8, ex.w_packed.shape[2], dtype=torch.int32, device=dev)
    sc_pad = torch.full((3, n + 8, ex.scales.shape[2]), float("nan"), dtype=TORCH_DTYPE[dtype], device=dev)
    bi_pad = sc_pad.clone()
    words_pad[:, :n] = ex.w_packed
    sc_pad[:, :n] = ex.scales
    bi_pad[:, :n] = ex.biases
    exp = q.ExpertWeights(words_pad[:, :n], sc_pad[:, :n], bi_pad[:, :n], n, k, gs, bits)
    idx = torch.tensor([2, -1, 0, 3, 1], dtype=torch.int32, device=dev)
    x = synth.normal_x((5, k), dtype, seed=72).to(dev)
    y = q.gather_qmv(x, exp, idx)
    torch.cuda.synchronize()
    yv = values(y)
    assert np.isnan(yv[1]).all() and np.isnan(yv[3]).all()
    ref = O.gather_reference(values(x), _oracle_triples(ws), idx.cpu().numpy(), k, gs, bits, dtype)
    good = [0, 2, 4]
    res = O.check(yv[good], ref["y_ref"][good], ref["tol"][good])
    assert res["ok"], res


def test_gather_qmv_errors():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    ex, _ = _experts(64, 256, 64, 4, "bf16", 2, 730, dev)
    x = synth.normal_x((3, 256), "bf16", seed=73).to(dev)
    idx = torch.zeros(3, dtype=torch.int32, device=dev)
    buf = synth.normal_x((2, 6, 256), "bf16", seed=74).to(dev)
    with pytest.raises(q.QmmError) as e:   # rows that do not fold into one level
        q.gather_qmv(buf[:, :3], ex, torch.zeros(6, dtype=torch.int32, device=dev))
    assert e.value.code == -4
    with pytest.raises(ValueError):        # one index per row
        q.gather_qmv(buf[0], ex, idx)
    y = torch.zeros(0, 64, dtype=torch.bfloat16, device=dev)
    q.gather_qmv(x[:0], ex, idx[:0], out=y)    # zero rows: no-op


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_dequantize_bit_exact(bits, dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    for gs, n, k in ((32, 37, 96), (64, 130, 320), (128, 5, 1024)):
        w = synth.normal_weight(n, k, 0.02, seed=800 + bits + gs).numpy()
        qz = O.quantize(w, gs, bits, dtype)
        qw = upload_oracle_weight(qz, dev)
        out = torch.full((n, k + 8), float("nan"), dtype=TORCH_DTYPE[dtype], device=dev)
        q.dequantize(qw, out=out[:, :k])
        torch.cuda.synchronize()
        expect = O.dequantize_dtype(qz["codes"], qz["scales_bits"], qz["biases_bits"], gs, dtype)
        got = half_bits(out)
        assert np.array_equal(got[:, :k], expect), (bits, gs, dtype)
        assert np.isnan(values(out[:, k:])).all()   # the row padding is untouched


@pytest.mark.parametrize("bits,dtype", [(4, "bf16"), (8, "fp16"), (3, "bf16")])
def test_embedding_rows_bit_exact_and_bad_indices(bits, dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k, gs = 300, 256, 64
    w = synth.normal_weight(n, k, 0.5, seed=900 + bits).numpy()
    qz = O.quantize(w, gs, bits, dtype)
    qw = upload_oracle_weight(qz, dev)
    idx_list = [5, 299, 0, 5, 300, -1, 123]
    idx = torch.tensor(idx_list, dtype=torch.int32, device=dev)
    out = q.embedding(qw, idx)
    torch.cuda.synchronize()
    rows = O.embedding_reference(O.pack(qz["codes"], bits), qz["scales_bits"], qz["biases_bits"], idx_list, k, gs,
                                 bits, dtype)
    got = half_bits(out)
    for r, ref in enumerate(rows):
        if ref is None:
            assert np.isnan(values(out[r])).all(), r
        else:
            assert np.array_equal(got[r], ref), r
    assert q.embedding(qw, idx[:0]).shape == (0, k)


@pytest.mark.parametrize("m,n,bits,dtype", [(32, 3001, 4, "bf16"), (5, 777, 8, "fp16"), (17, 130, 3, "bf16")])
def test_qmv_argmax_parity(m, n, bits, dtype):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    k, gs = 1024, 64
    w = synth.normal_weight(n, k, 0.02, seed=1000 + n).numpy()
    qz = O.quantize(w, gs, bits, dtype)
    qw = upload_oracle_weight(qz, dev)
    x = synth.normal_x((m, k), dtype, seed=1001).to(dev)
    idx, val, y = q.qmv_argmax(x, qw)
    idx2, val2, none = q.qmv_argmax(x, qw, logits=False)
    y_plain = q.qmv(x, qw)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))     # same logits as qmv
    assert torch.equal(idx, idx2) and torch.equal(val, val2)               # logits optional
    first = torch.argmax(y.float(), dim=1).to(torch.int32)                 # first maximum
    assert torch.equal(idx, first)
    assert torch.equal(val, y.float().gather(1, idx.long()[:, None])[:, 0])
    ref = O.reference(values(x), O.pack(qz["codes"], bits), qz["scales_bits"], qz["biases_bits"], k, gs, bits, dtype)
    ok = O.argmax_acceptable(ref["y_ref"], ref["tol"])
    for r in range(m):
        assert int(idx[r]) in ok[r], r


def test_qmv_argmax_ties_pick_first_and_nan():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k, gs, bits, dtype = 300, 512, 64, 4, "bf16"
    w = synth.normal_weight(n, k, 0.02, seed=1100).numpy()
    for r in (41, 7, 250):         # three identical, dominant rows: 7 must win
        w[r] = 1.0 + 0.01 * np.arange(k) / k
    qw = upload_oracle_weight(O.quantize(w, gs, bits, dtype), dev)
    x = torch.ones(3, k, dtype=torch.bfloat16, device=dev)
    x[2, 5] = float("nan")         # a NaN row: every logit NaN, the first one wins
    idx, val, y = q.qmv_argmax(x, qw)
    torch.cuda.synchronize()
    assert idx[:2].tolist() == [7, 7]
    assert int(idx[2]) == 0 and bool(torch.isnan(val[2]))


def test_qmv_argmax_lm_head_full_size():
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    c = synth.LM_HEAD
    w = synth.normal_weight(c["n"], c["k"], c["w_std"], seed=c["w_seed"]).to(dev)
    qw = q.quantize(w, c["group_size"], c["bits"], c["dtype"])
    x = synth.normal_x((c["m"], c["k"]), c["dtype"], seed=c["x_seed"]).to(dev)
    idx, val, y = q.qmv_argmax(x, qw)
    torch.cuda.synchronize()
    assert torch.equal(idx, torch.argmax(y.float(), dim=1).to(torch.int32))
    # the chosen columns against the oracle, one by one
    rows = sorted(set(idx.tolist()))
    from qmm_testlib import reference_rows
    ref = reference_rows(values(x), qw, c["dtype"], rows=rows)
    for r in range(c["m"]):
        j = rows.index(int(idx[r]))
        assert abs(float(val[r]) - ref["y_ref"][r, j]) <= ref["tol"][r, j]


def test_qmv_argmax_chunked_activations():
    # 20 rows x K = 4096 do not fit in LDS at once: the chunked decode kernel runs
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k, gs, bits, dtype = 1500, 4096, 128, 4, "bf16"
    w = synth.normal_weight(n, k, 0.02, seed=1200).numpy()
    qz = O.quantize(w, gs, bits, dtype)
    qw = upload_oracle_weight(qz, dev)
    x = synth.normal_x((20, k), dtype, seed=1201).to(dev)
    idx, val, y = q.qmv_argmax(x, qw)
    torch.cuda.synchronize()
    assert torch.equal(idx, torch.argmax(y.float(), dim=1).to(torch.int32))
    ref = O.reference(values(x), O.pack(qz["codes"], bits), qz["scales_bits"], qz["biases_bits"], k, gs, bits, dtype)
    assert_close(y, ref, "chunked qmv")
    ok = O.argmax_acceptable(ref["y_ref"], ref["tol"])
    assert all(int(idx[r]) in ok[r] for r in range(20))


def test_qmv_argmax_workspace_reuse_and_graph_replay():
    """One zero-filled workspace serves calls of different row counts (stream and chunked
    kernels) and is all-zero after each; a captured call replays to the eager result."""
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    ws = q.argmax_workspace(32, dev)
    for k, n in ((1024, 3001), (4096, 1500)):
        qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=1300 + k).to(dev), 128, 4, "bf16")
        for m in (32, 5, 17, 1, 32):
            x = synth.normal_x((m, k), "bf16", seed=1301 + m).to(dev)
            idx, val, y = q.qmv_argmax(x, qw, workspace=ws)
            fresh = q.qmv_argmax(x, qw)
            torch.cuda.synchronize()
            assert not ws.any(), (k, m)
            assert torch.equal(idx, fresh[0]) and torch.equal(val, fresh[1]), (k, m)
            assert torch.equal(idx, torch.argmax(y.float(), dim=1).to(torch.int32)), (k, m)
    qw = q.quantize(synth.normal_weight(3001, 1024, 0.02, seed=1310).to(dev), 64, 4, "bf16")
    x = synth.normal_x((32, 1024), "bf16", seed=1311).to(dev)
    idx = torch.empty(32, dtype=torch.int32, device=dev)
    val = torch.empty(32, dtype=torch.float32, device=dev)
    y = torch.empty(32, 3001, dtype=torch.bfloat16, device=dev)
    eager = q.qmv_argmax(x, qw, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qmv_argmax(x, qw, workspace=ws, out=y, out_index=idx, out_value=val)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qmv_argmax(x, qw, workspace=ws, out=y, out_index=idx, out_value=val)
    for rep in range(4):
        idx.fill_(-1)
        val.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, eager[0]) and torch.equal(val, eager[1]) and torch.equal(y, eager[2]), rep
        assert not ws.any(), rep
        x2 = synth.normal_x((32, 1024), "bf16", seed=rep).to(dev)      # eager work between replays
        q.qmv_argmax(x2, qw, workspace=ws)
        torch.cuda.synchronize()
