"""Run-to-run determinism of the decode kernels: identical calls must give identical bits
(a kernel that reads uninitialized LDS, registers or output memory fails this)."""
import pytest
import torch

import synth
from qmm_testlib import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_repeated_calls_bitwise_equal(dtype, bits):
    import bit_affine_quantized_qmv_amd as q
    dev = require_gpu()
    n, k = 1000, 640
    for gs in (32, 64, 128):
        qw = q.quantize(synth.normal_weight(n, k, 1.0, seed=bits * 7 + gs).to(dev), gs, bits, dtype)
        for m in (1, 16, 17, 32):
            x = synth.normal_x((m, k), dtype, seed=m).to(dev)
            ref = q.qmv(x, qw).clone()
            for _ in range(12):
                # scribble over the output buffer the allocator will hand back next
                junk = torch.full_like(ref, float("nan"))
                del junk
                y = q.qmv(x, qw)
                assert torch.equal(y, ref), (dtype, bits, gs, m)
