"""GPU parity on the pages' workloads (synthetic values, the pages' shapes), including the
full-size decode (lm_head) and prefill cases in the launch configuration the benchmark
times.  Full-size outputs are checked against the oracle on sampled weight rows and then on
every output, weight rows taken in slices."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import (TORCH_DTYPE, assert_close, gather, half_bits, oracle_view_of, reference_rows,
                         require_gpu, upload_oracle_weight, values, words)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _assert_quantize_exact(qw, w_np, gs, bits, dtype):
    ref = O.quantize(w_np, gs, bits, dtype)
    assert np.array_equal(half_bits(qw.scales), ref["scales_bits"])
    assert np.array_equal(half_bits(qw.biases), ref["biases_bits"])
    assert np.array_equal(words(qw.w_packed), O.pack(ref["codes"], bits))


def test_probe_workload(dev):
    """issue-47331 probe: K=2048, N=1024, 4-bit, group 64, bf16; x in [2,K], [2,1,K],
    [2,4,K].  Every row within the bound; the page metric inside the printed band."""
    import bit_affine_quantized_qmv_amd as q
    with open(os.path.join(GOLDEN, "probe_band.json")) as f:
        band = json.load(f)["band"]
    w = synth.probe_weight()
    qw = q.quantize(w.to(dev), 64, 4, "bf16")
    _assert_quantize_exact(qw, w.numpy(), 64, 4, "bf16")
    k = 2048
    s32_ref = O.quantize(w.numpy(), 64, 4, "bf16")
    g = np.arange(k) // 64
    w_page = s32_ref["s32"][:, g].astype(np.float64) * s32_ref["codes"] + s32_ref["b32"][:, g]
    for i, shape in enumerate([(2, k), (2, 1, k), (2, 4, k)]):
        x = synth.normal_x(shape, "bf16", seed=1 + i).to(dev)
        y = q.qmm_t(x, qw)
        assert y.shape == tuple(shape[:-1]) + (1024,)
        assert torch.equal(y, q.qmv(x, qw))
        rows = values(x).reshape(-1, k)
        assert_close(y.reshape(-1, 1024), reference_rows(rows, qw, "bf16"), str(shape))
        metric = O.page_metric(values(y).reshape(-1, 1024), rows @ w_page.T)
        assert np.all((metric > band[0]) & (metric < band[1])), (shape, metric)


@pytest.mark.parametrize("i", range(len(synth.DECODE_SHAPES)))
@pytest.mark.parametrize("bits", [4, 8])
def test_batched_decode_workload(dev, i, bits):
    """Batched decode projections, B in {1..32}: the bound, and row i of every batched call
    equal to the B=1 call on that row, bit for bit."""
    import bit_affine_quantized_qmv_amd as q
    k, n = synth.DECODE_SHAPES[i]
    w = synth.normal_weight(n, k, 0.02, seed=100 + i)
    qw = q.quantize(w.to(dev), 64, bits, "bf16")
    _assert_quantize_exact(qw, w.numpy(), 64, bits, "bf16")
    x = synth.normal_x((32, 1, k), "bf16", seed=200 + i).to(dev)
    y1 = [q.qmv(x[r:r + 1], qw) for r in range(32)]
    for b in synth.DECODE_BATCHES:
        y = q.qmv(x[:b], qw)
        for r in range(b):
            assert torch.equal(y[r], y1[r][0]), (b, r)
    assert_close(q.qmv(x, qw).reshape(32, n), reference_rows(values(x).reshape(32, k), qw, "bf16"))
    buf = synth.normal_x((64, 1, k), "bf16", seed=300 + i).to(dev)
    y_even = q.qmv(buf[0::2], qw)
    assert torch.equal(y_even, q.qmv(buf[0::2].contiguous(), qw))


ODD_CASES = [(n, b, gs, dt) for n in synth.ODD_N for b in synth.ODD_BITS for gs in synth.GROUPS
             for dt in ("fp16", "bf16")]


@pytest.mark.parametrize("case", range(len(ODD_CASES)))
def test_odd_n_running_sum_workload(dev, case):
    """Odd N with K=4096 and x alternating 2048, 1: the bound on every row, and the rows
    whose dequantized weights are all exactly zero must come out exactly zero (a running
    sum of x kept in half precision would make them large)."""
    import bit_affine_quantized_qmv_amd as q
    n, bits, gs, dtype = ODD_CASES[case]
    k = 4096
    x = synth.alternating_x(k, dtype).to(dev)
    for first_zero in ((False, True) if n == 1 else (False,)):
        c = synth.odd_n_weight(n, k, bits, gs, seed=400 + case, first_row_zero=first_zero)
        qo = {"codes": c["codes"], "scales_bits": O.to_dtype_bits(c["scale_values"], dtype),
              "biases_bits": O.to_dtype_bits(c["bias_values"], dtype), "bits": bits,
              "group_size": gs, "dtype": dtype}
        qw = upload_oracle_weight(qo, dev)
        y = q.qmv(x, qw)
        ref = reference_rows(values(x), qw, dtype)
        assert_close(y, ref, ODD_CASES[case])
        yz = values(y)[0, c["zero_rows"]]
        assert np.all(yz == 0), (ODD_CASES[case], yz[:8])


def _assert_all_outputs(y2d, x_rows, qw, dtype, slice_rows, what):
    """Every output of a full-size call against the oracle, weight rows taken in slices."""
    n = y2d.shape[1]
    ov = oracle_view_of(qw)   # the weight copied to the host once
    y_host = y2d.cpu()
    for lo in range(0, n, slice_rows):
        rows = np.arange(lo, min(n, lo + slice_rows))
        ref = O.reference(x_rows, ov["w_packed"], ov["scales_bits"], ov["biases_bits"], qw.K, qw.group_size,
                          qw.bits, dtype, rows=rows)
        assert_close(y_host[:, lo:lo + len(rows)], ref, "%s, weight rows %d.." % (what, lo))


def test_lm_head_full_size(dev):
    """lm_head decode at full size (x [32,1,1024], W [151936,1024], 4-bit, group 64, bf16):
    the GPU quantizer is bit-exact; the folded and the forced per-batch-element launches
    agree bit for bit; sampled weight rows satisfy the bound for all 32 activation rows."""
    import bit_affine_quantized_qmv_amd as q
    cfg = synth.LM_HEAD
    w = synth.normal_weight(cfg["n"], cfg["k"], cfg["w_std"], seed=cfg["w_seed"])
    qw = q.quantize(w.to(dev), cfg["group_size"], cfg["bits"], cfg["dtype"])
    _assert_quantize_exact(qw, w.numpy(), cfg["group_size"], cfg["bits"], cfg["dtype"])
    del w
    x = synth.normal_x((cfg["m"], 1, cfg["k"]), cfg["dtype"], seed=cfg["x_seed"]).to(dev)
    y = q.qmv(x, qw)
    y_forced = q.qmv(x, qw, flags=q.QMM_FLAG_FORCE_STRIDED)
    assert torch.equal(y, y_forced)
    rows = synth.rows_sample(cfg["n"], 1024, seed=1)
    ref = reference_rows(values(x).reshape(cfg["m"], cfg["k"]), qw, cfg["dtype"], rows=rows)
    assert_close(y.reshape(cfg["m"], cfg["n"])[:, rows], ref, "lm_head")
    y1 = q.qmv(x[5], qw)
    assert torch.equal(y1[0], y[5, 0])
    _assert_all_outputs(y.reshape(cfg["m"], cfg["n"]), values(x).reshape(cfg["m"], cfg["k"]), qw, cfg["dtype"],
                        19000, "lm_head all outputs")


def test_prefill_full_size(dev):
    """Prefill at full size (x [4,512,4096] and a narrowed view of [4,1024,4096],
    W [14336,4096], 4-bit, group 128, bf16): bit-exact quantizer, view == contiguous copy
    bit for bit (start 0 and 256), sampled weight rows within the bound for every row."""
    import bit_affine_quantized_qmv_amd as q
    cfg = synth.PREFILL
    w = synth.normal_weight(cfg["n"], cfg["k"], cfg["w_std"], seed=cfg["w_seed"])
    qw = q.quantize(w.to(dev), cfg["group_size"], cfg["bits"], cfg["dtype"])
    _assert_quantize_exact(qw, w.numpy(), cfg["group_size"], cfg["bits"], cfg["dtype"])
    del w
    shape = (cfg["b"], cfg["s"], cfg["k"])
    x = synth.normal_x(shape, cfg["dtype"], seed=cfg["x_seed"]).to(dev)
    y = q.qmm_t(x, qw)
    rows = synth.rows_sample(cfg["n"], 192, seed=2)
    ref = reference_rows(values(x).reshape(-1, cfg["k"]), qw, cfg["dtype"], rows=rows)
    assert_close(y.reshape(-1, cfg["n"])[:, rows], ref, "prefill contiguous")
    _assert_all_outputs(y.reshape(-1, cfg["n"]), values(x).reshape(-1, cfg["k"]), qw, cfg["dtype"], 2048,
                        "prefill all outputs")
    buf = synth.normal_x((cfg["b"], 2 * cfg["s"], cfg["k"]), cfg["dtype"], seed=cfg["buf_seed"]).to(dev)
    for start in (0, 256):
        view = buf[:, start:start + cfg["s"], :]
        assert view.stride() == (2 * cfg["s"] * cfg["k"], cfg["k"], 1)
        yv = q.qmm_t(view, qw)
        assert torch.equal(yv, q.qmm_t(view.contiguous(), qw)), start
        if start == 0:
            refv = reference_rows(gather(buf, view), qw, cfg["dtype"], rows=rows)
            assert_close(yv.reshape(-1, cfg["n"])[:, rows], refv, "prefill view")
