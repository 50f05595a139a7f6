"""GPU parity for activation layouts the dispatcher accepts but the workload tests do not
reach: broadcast (stride-0) batch dims in decode and prefill, every batch element checked
against the oracle (candle pitfall page "Metal 上批量 matmul 结果不对", section 怎么确认没中招:
check every batch element, not only the first), the quick-reproduction shape of MLX pull
request 4516 ("Validation and quick reproduction": K = 2560, one output feature, 8-bit
codes, group 64), and run-to-run determinism on every decode kernel path."""
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import assert_close, gather, reference_rows, require_gpu, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _quantized(q, dev, n, k, gs, bits, dtype, seed, std=1.0):
    return q.quantize(synth.normal_weight(n, k, std, seed=seed).to(dev), gs, bits, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("bits", [4, 8, 3])
def test_broadcast_rows_decode(dev, dtype, bits):
    """x.expand over a batch dim (stride 0): one level of 8 identical rows, and two levels
    [4, 3, K] with batch stride 0.  Every row within the bound (the oracle gathers the rows
    from the base storage through the view's strides) and equal, bit for bit, to the call
    on the base row alone."""
    import bit_affine_quantized_qmv_amd as q
    n, k, gs = 300, 512, 64
    qw = _quantized(q, dev, n, k, gs, bits, dtype, seed=60 + bits)
    base = synth.normal_x((1, k), dtype, seed=61).to(dev)
    x1 = base.expand(8, k)
    assert x1.stride() == (0, 1)
    y1 = q.qmv(x1, qw)
    assert_close(y1, reference_rows(gather(base, x1), qw, dtype), "expand 8")
    y_base = q.qmv(base, qw)
    for r in range(8):
        assert torch.equal(y1[r], y_base[0]), r
    base3 = synth.normal_x((1, 3, k), dtype, seed=62).to(dev)
    x2 = base3.expand(4, 3, k)
    assert x2.stride() == (0, k, 1)
    y2 = q.qmv(x2, qw)
    assert y2.shape == (4, 3, n)
    assert_close(y2.reshape(12, n), reference_rows(gather(base3, x2), qw, dtype), "expand 4x3")
    y_b3 = q.qmv(base3[0], qw)
    for b in range(4):
        assert torch.equal(y2[b], y_b3), b


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_broadcast_rows_prefill(dev, dtype):
    """Prefill with a stride-0 batch dim: x = base.expand(4, 160, K) (640 rows through the
    MFMA kernel).  Every row within the bound, each batch element equal to the call on the
    base rows, bit for bit."""
    import bit_affine_quantized_qmv_amd as q
    n, k, gs = 264, 768, 128
    qw = _quantized(q, dev, n, k, gs, 4, dtype, seed=63)
    base = synth.normal_x((1, 160, k), dtype, seed=64).to(dev)
    x = base.expand(4, 160, k)
    assert x.stride() == (0, k, 1)
    y = q.qmm_t(x, qw)
    assert_close(y.reshape(640, n), reference_rows(gather(base, x), qw, dtype), "prefill expand")
    y_base = q.qmm_t(base[0], qw)
    for b in range(4):
        assert torch.equal(y[b], y_base), b


@pytest.mark.parametrize("rows", [1, 4, 32])
def test_pr_reproduction_shape(dev, rows):
    """K = 2560, N = 1, 8-bit codes, group 64, bf16 (the pull request's quick reproduction):
    within the bound, and row i of the batched call equal to the single-row call."""
    import bit_affine_quantized_qmv_amd as q
    k, n = 2560, 1
    qw = _quantized(q, dev, n, k, 64, 8, "bf16", seed=65, std=0.02)
    x = synth.normal_x((rows, 1, k), "bf16", seed=66).to(dev)
    y = q.qmv(x, qw)
    assert y.shape == (rows, 1, 1)
    assert_close(y.reshape(rows, 1), reference_rows(values(x).reshape(rows, k), qw, "bf16"), "K=2560 N=1")
    for r in range(rows):
        assert torch.equal(q.qmv(x[r], qw)[0], y[r, 0]), r


# Shapes that reach each decode kernel path: whole rows per wave (wide weights), rows cut
# into parts (narrower weights or long K), activations too large for LDS (K processed in
# chunks), and 17-32 rows at long K (two 16-row blocks).
DET_CASES = [
    # (bits, gs, k, n, rows)
    (4, 64, 1024, 2000, 32),
    (4, 64, 2048, 1000, 8),
    (4, 64, 3072, 1000, 32),
    (8, 64, 1024, 1000, 16),
    (8, 32, 1408, 700, 32),
    (4, 32, 4096, 600, 32),
    (4, 128, 8192, 500, 16),
    (2, 32, 640, 1000, 16),
    (6, 32, 640, 1000, 1),
    (5, 64, 4096, 500, 32),
    (4, 64, 1024, 65000, 32),    # whole rows per wave (streaming kernel)
    (6, 32, 640, 65000, 16),
    (2, 32, 640, 65000, 1),
    (5, 64, 1024, 65000, 32),
]


@pytest.mark.parametrize("case", range(len(DET_CASES)))
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_repeated_calls_bitwise_equal_all_paths(dev, case, dtype):
    """Identical calls give identical bits on every decode path (a kernel that reads
    uninitialized LDS, registers or output memory, or races between waves, fails this)."""
    import bit_affine_quantized_qmv_amd as q
    bits, gs, k, n, rows = DET_CASES[case]
    qw = _quantized(q, dev, n, k, gs, bits, dtype, seed=70 + case)
    x = synth.normal_x((rows, k), dtype, seed=71 + case).to(dev)
    ref = q.qmv(x, qw).clone()
    assert_close(ref, reference_rows(values(x), qw, dtype), DET_CASES[case])
    for _ in range(8):
        junk = torch.full_like(ref, float("nan"))
        del junk
        y = q.qmv(x, qw)
        assert torch.equal(y, ref), (DET_CASES[case], dtype)


@pytest.mark.parametrize("n", [262144, 327680])
def test_decode_many_pairs_per_wave(dev, n):
    """Weights long enough that each wave of the full decode grid (256 compute units) holds
    four or five 32-row tile pairs (K = 1024, 4-bit, group 64, 32 activation rows): four
    pairs' outputs fit the waves' LDS area and are stored after the weight stream, five do
    not and are stored pair by pair.  Sampled weight rows (the last 64 included) within the
    bound for all 32 rows, and rows 0, 17 and 31 bitwise equal to their one-row calls."""
    import numpy as np
    import bit_affine_quantized_qmv_amd as q
    k, gs, bits, dtype = 1024, 64, 4, "bf16"
    words, sc, bi = synth.random_packed_weight(n, k * bits // 32, k // gs, dtype, seed=1300 + n % 1000)
    qw = q.QuantizedWeight(words.to(dev), sc.to(dev), bi.to(dev), n, k, gs, bits)
    x = synth.normal_x((32, k), dtype, seed=1301).to(dev)
    y = q.qmv(x, qw)
    rows = np.unique(np.concatenate([synth.rows_sample(n, 768, seed=3), np.arange(n - 64, n)]))
    ref = reference_rows(values(x), qw, dtype, rows=rows)
    assert_close(y[:, rows], ref, "many pairs per wave, N=%d" % n)
    for r in (0, 17, 31):
        assert torch.equal(q.qmv(x[r:r + 1], qw)[0], y[r]), (n, r)


@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (8, 32), (8, 64)])
@pytest.mark.parametrize("m", [1, 32])
def test_decode_scales_two_bytes_off_alignment(dev, bits, gs, m):
    """Scales and biases whose arrays start one halfword past a 4-byte boundary (views one
    element into a buffer; rows of whole slots, so only the bases are off): the kernels read
    them one halfword at a time, and the outputs are bitwise those of the same values at
    aligned addresses and within the bound."""
    import bit_affine_quantized_qmv_amd as q
    n, k, dtype = 2000, 1024, "bf16"
    g = k // gs
    words, sc, bi = synth.random_packed_weight(n, k * bits // 32, g, dtype, seed=1400 + 10 * bits + gs)
    qw = q.QuantizedWeight(words.to(dev), sc.to(dev), bi.to(dev), n, k, gs, bits)
    sbuf = torch.zeros(n * g + 1, dtype=sc.dtype, device=dev)
    bbuf = torch.zeros(n * g + 1, dtype=bi.dtype, device=dev)
    sbuf[1:] = sc.reshape(-1).to(dev)
    bbuf[1:] = bi.reshape(-1).to(dev)
    qw_off = q.QuantizedWeight(qw.w_packed, sbuf[1:].view(n, g), bbuf[1:].view(n, g), n, k, gs, bits)
    assert qw_off.scales.data_ptr() % 4 == 2 and qw_off.biases.data_ptr() % 4 == 2
    x = synth.normal_x((m, k), dtype, seed=1401).to(dev)
    y = q.qmv(x, qw)
    y_off = q.qmv(x, qw_off)
    assert torch.equal(y, y_off), (bits, gs, m)
    assert_close(y_off, reference_rows(values(x), qw, dtype), "scales off alignment")
