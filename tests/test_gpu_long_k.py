"""GPU parity of decode at long K with few activation rows.  A single-row call stages only
that row in LDS, so it runs the streaming or parts kernels up to K of about 64K; 2-8 rows
whose 16-row staging does not fit stage 8 rows, and the rest take the chunked kernel.  Each case is checked against
the oracle, and every row of the call bit for bit against the same row called alone (the
arithmetic of a row does not depend on how many rows share the call or which kernel runs
it; mlx pull request 4516, "Correctness": bitwise identical results across batch sizes)."""
import pytest
import torch

import synth
from qmm_testlib import assert_close, reference_rows, require_gpu, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


LONG_K_CASES = [
    # (bits, gs, k, n, rows, dtype)
    (4, 128, 8192, 700, 1, "bf16"),
    (4, 64, 8192, 700, 3, "bf16"),
    (8, 64, 8192, 500, 8, "fp16"),
    (4, 32, 16384, 300, 2, "bf16"),
    (3, 64, 8192, 300, 5, "bf16"),
    (6, 32, 12288, 200, 1, "fp16"),
    (4, 64, 65536, 64, 1, "bf16"),
    (4, 128, 4224, 1000, 7, "bf16"),   # K past 4096, 16 staged rows just fit
]


@pytest.mark.parametrize("case", range(len(LONG_K_CASES)))
def test_long_k_few_rows(dev, case):
    import bit_affine_quantized_qmv_amd as q
    bits, gs, k, n, rows, dtype = LONG_K_CASES[case]
    qw = q.quantize(synth.normal_weight(n, k, 1.0, seed=150 + case).to(dev), gs, bits, dtype)
    x = synth.normal_x((rows, k), dtype, seed=151 + case).to(dev)
    y = q.qmv(x, qw)
    assert_close(y, reference_rows(values(x), qw, dtype), LONG_K_CASES[case])
    for r in range(rows):
        assert torch.equal(q.qmv(x[r:r + 1], qw)[0], y[r]), (LONG_K_CASES[case], r)
    assert torch.equal(q.qmv(x, qw), y)   # repeated call, same bits


@pytest.mark.parametrize("k,gs,rows", [(4096, 128, 1), (4096, 128, 2), (4096, 128, 3), (8192, 64, 1),
                                       (4096, 128, 17), (8192, 64, 5)])
def test_argmax_with_few_staged_rows(dev, k, gs, rows):
    """The fused argmax when one activation row is staged: its 8-byte LDS keys follow the
    per-group sums, whose float count (K / gs + 3 per staged row) can be odd, and must still
    be 8-byte aligned for the 64-bit LDS atomics (17 rows: the second 16-row pass has one)."""
    import bit_affine_quantized_qmv_amd as q
    qw = q.quantize(synth.normal_weight(1500, k, 0.02, seed=170 + rows).to(dev), gs, 4, "bf16")
    x = synth.normal_x((rows, k), "bf16", seed=171 + rows).to(dev)
    ws = q.argmax_workspace(rows, dev)
    idx, val, y = q.qmv_argmax(x, qw, workspace=ws)
    torch.cuda.synchronize()
    assert not ws.any()
    assert torch.equal(y, q.qmv(x, qw))
    assert torch.equal(idx, torch.argmax(y.float(), dim=1).to(torch.int32))
    assert torch.equal(val, y.float().gather(1, idx.long()[:, None])[:, 0])
