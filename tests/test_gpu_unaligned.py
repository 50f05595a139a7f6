"""GPU parity of the unaligned-K path: K a multiple of the group size but not of 128 (the
decode kernels mask a last slot that ends past K; the MFMA kernel masks its last k step),
and weight rows padded to word counts the decode kernels do not take, which run the MFMA
kernel at every row count (MLX pull request 4516, second commit text: inputs that are not
aligned for the fast qmv kernel take the generic kernel and its guarded tail)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import TORCH_DTYPE, assert_close, reference_rows, require_gpu, upload_oracle_weight, values

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 8]
DT = ["bf16", "fp16"]
# (K, group_size): a single group, partial last steps of 32, K a multiple of 64 but not 128
SHAPES = [(32, 32), (96, 32), (160, 32), (1056, 32), (1088, 64), (4128, 32)]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _weight(n, k, seed):
    return np.random.default_rng(seed).standard_normal((n, k)).astype(np.float32)


def _padded(qw, extra):
    """The same weight with every code row padded by `extra` words (a strided view)."""
    import bit_affine_quantized_qmv_amd as q
    n, words = qw.w_packed.shape
    buf = torch.full((n, words + extra), -1, dtype=torch.int32, device=qw.w_packed.device)
    buf[:, :words] = qw.w_packed
    return q.QuantizedWeight(buf[:, :words], qw.scales, qw.biases, qw.N, qw.K, qw.group_size, qw.bits)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dtype", DT)
def test_unaligned_k_parity(dev, bits, dtype):
    import bit_affine_quantized_qmv_amd as q
    n = 333
    for k, gs in SHAPES:
        qw = upload_oracle_weight(O.quantize(_weight(n, k, bits * 11 + k), gs, bits, dtype), dev)
        for m in (1, 7, 32, 33, 130):
            x = synth.normal_x((m, k), dtype, seed=m + k).to(dev)
            y = q.qmm_t(x, qw)
            assert_close(y, reference_rows(values(x), qw, dtype), "K=%d gs=%d m=%d" % (k, gs, m))
            if m <= 32:
                assert torch.equal(q.qmv(x, qw), y), (k, m)


@pytest.mark.parametrize("k,gs", [(1056, 32), (4128, 32), (1088, 64), (96, 32)])
def test_unaligned_batch_invariance(dev, k, gs):
    """Row i of every [B, 1, K] decode call (B = 1..32) equals the single-row call bit for
    bit at unaligned K, also across the change from the streaming to the chunked decode
    kernel (K = 4128 at B > 16), through a strided batch and the forced per-row plan."""
    import bit_affine_quantized_qmv_amd as q
    n = 1000
    for bits in (4, 8, 3):
        qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=bits + k).to(dev), gs, bits, "bf16")
        x = synth.normal_x((32, 1, k), "bf16", seed=bits).to(dev)
        singles = [q.qmv(x[i], qw) for i in range(32)]
        for b in (1, 2, 16, 17, 32):
            y = q.qmv(x[:b], qw)
            for i in range(b):
                assert torch.equal(y[i], singles[i]), (bits, b, i)
        assert torch.equal(q.qmv(x, qw, flags=q.QMM_FLAG_FORCE_STRIDED), q.qmv(x, qw))
        buf = synth.normal_x((64, k), "bf16", seed=99).to(dev)
        assert torch.equal(q.qmv(buf[0::2], qw), q.qmv(buf[0::2].contiguous(), qw))
        assert_close(q.qmv(x, qw).view(32, n), reference_rows(values(x).reshape(32, k), qw, "bf16"),
                     "bits=%d" % bits)


@pytest.mark.parametrize("bits,extra", [(3, 1), (5, 3), (6, 2), (2, 2), (4, 4)])
def test_padded_row_strides(dev, bits, extra):
    """Rows padded to a word count that is not a multiple of 4 (3-, 5-bit: any; 2-, 6-bit:
    even) run the MFMA kernel at K = 1024; a padding of 4 words keeps the decode kernels.
    Either way the padding words (all ones) are never read into a result."""
    import bit_affine_quantized_qmv_amd as q
    n, k, gs = 517, 1024, 64
    qw = upload_oracle_weight(O.quantize(_weight(n, k, bits), gs, bits, "fp16"), dev)
    qp = _padded(qw, extra)
    for m in (1, 9, 40):
        x = synth.normal_x((m, k), "fp16", seed=m).to(dev)
        y = q.qmm_t(x, qp)
        assert_close(y, reference_rows(values(x), qw, "fp16"), "bits=%d m=%d" % (bits, m))
        if m <= 32:
            assert torch.equal(q.qmv(x, qp), y)
    dense_rows = (k * bits // 32) % 4 == 0
    if not dense_rows or extra % 4 == 0:
        return
    # a padded weight and a differently padded copy run the same kernel: same bits
    x = synth.normal_x((5, k), "fp16", seed=5).to(dev)
    assert torch.equal(q.qmv(x, qp), q.qmv(x, _padded(qw, extra + 4)))


def test_unaligned_every_output_written_and_no_spill(dev):
    import bit_affine_quantized_qmv_amd as q
    n, k = 203, 96
    qw = q.quantize(synth.normal_weight(n, k, 1.0, seed=9).to(dev), 32, 5, "bf16")
    for m in (1, 7, 32, 45, 300):
        guard = 4096
        raw = torch.full((guard * 2 + m * n,), 12345.0, dtype=torch.bfloat16, device=dev)
        y = raw[guard:guard + m * n].view(m, n)
        y.fill_(float("nan"))
        x = synth.normal_x((m, k), "bf16", seed=m).to(dev)
        q.qmm_t(x, qw, out=y)
        assert not torch.isnan(y).any(), m
        assert (raw[:guard] == 12345.0).all() and (raw[guard + m * n:] == 12345.0).all(), m


def test_full_size_unaligned_sampled(dev):
    """A decode-sized call at K = 4096 + 32 (gs 32, 4-bit, N = 14336), sampled rows against
    the oracle, plus a 512-row prefill of the same weight."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 14336, 4128
    qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=4).to(dev), 32, 4, "bf16")
    rows = synth.rows_sample(n, 256, seed=4)
    for m in (1, 512):
        x = synth.normal_x((m, k), "bf16", seed=m).to(dev)
        y = q.qmm_t(x, qw)
        xm = values(x)[: min(m, 8)]
        assert_close(y[: min(m, 8), rows], reference_rows(xm, qw, "bf16", rows=rows), "m=%d" % m)


def test_gathered_and_argmax_at_unaligned_k(dev):
    """The gathered and argmax decode forms run at unaligned K (equal to qmv per row); rows
    padded to a word count the decode kernels cannot take are refused there."""
    import bit_affine_quantized_qmv_amd as q
    k, n = 1056, 700
    qa = q.quantize(synth.normal_weight(n, k, 0.5, seed=1).to(dev), 32, 4, "bf16")
    qb = q.quantize(synth.normal_weight(n, k, 0.5, seed=2).to(dev), 32, 4, "bf16")
    x = synth.normal_x((5, k), "bf16", seed=2).to(dev)
    idx, val, y = q.qmv_argmax(x, qa)
    assert torch.equal(y, q.qmv(x, qa))
    assert torch.equal(idx, torch.argmax(y.float(), dim=1).to(torch.int32))
    ex = q.ExpertWeights.stack([qa, qb])
    sel = torch.tensor([1, 0, 1, 1, 0], dtype=torch.int32, device=dev)
    yg = q.gather_qmv(x, ex, sel)
    for r, e in enumerate(sel.tolist()):
        assert torch.equal(yg[r], q.qmv(x[r:r + 1], (qa, qb)[e])[0]), r
    aligned = q.quantize(synth.normal_weight(64, 1024, 0.5, seed=1).to(dev), 32, 3, "bf16")
    with pytest.raises(q.QmmError) as e:
        q.qmv_argmax(synth.normal_x((2, 1024), "bf16", seed=2).to(dev), _padded(aligned, 1))
    assert e.value.code == -5
    words = aligned.w_packed.shape[1]
    wp = torch.zeros(2, 64, words + 1, dtype=torch.int32, device=dev)[:, :, :words]
    wp[0] = aligned.w_packed
    wp[1] = aligned.w_packed
    ex_odd = q.ExpertWeights(wp, torch.stack([aligned.scales] * 2), torch.stack([aligned.biases] * 2), 64, 1024,
                             32, 3)
    with pytest.raises(q.QmmError) as e:
        q.gather_qmv(synth.normal_x((2, 1024), "bf16", seed=2).to(dev), ex_odd,
                     torch.zeros(2, dtype=torch.int32, device=dev))
    assert e.value.code == -5
