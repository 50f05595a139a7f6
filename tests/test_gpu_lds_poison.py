"""Results do not depend on what an earlier dispatch left in LDS.

A helper kernel (tests/lds_fill.hip) takes the whole LDS of every compute unit and fills
it with a pattern (bf16 and fp16 NaN pairs, all ones, zero, 0x5A5A5A5A) right before a
library call on the same stream.  A kernel that reads an LDS word it did not write in the
same launch (an activation or Σx pad, the argmax keys, the parts hand-off area, the top-k
histogram) then sees that pattern, and a NaN pattern spreads into the results even through
a multiply by zero.  Every call must give the same bits as without the fill.  The first
test shows that the fill reaches the next dispatch at all (the hardware does not clear LDS
between dispatches), so that the others are not vacuous.

Paths covered: the streaming decode kernel at one and two row tiles, the parts kernel, the
chunked kernel, the two 16-row blocks, every code width at the shapes with K = 640 and
group 32 in fp16, the fused argmax, the gathered form, both prefill kernels, and top-k with
and without column chunks."""
import ctypes
import os

import pytest
import torch

import synth
from qmm_testlib import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATTERNS = [0x7FC07FC0, 0x7E007E00, 0xFFFFFFFF, 0x00000000, 0x5A5A5A5A]
FILL_BLOCKS = 1024      # four whole-LDS workgroups per compute unit of a 256-CU device
PEEK_WORDS = 1024


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def helper(dev):
    path = os.path.join(ROOT, "tests", "_lds_fill.so")
    if not os.path.exists(path):
        raise RuntimeError("tests/_lds_fill.so is not built (build() compiles it)")
    lib = ctypes.CDLL(path)
    lib.lds_fill.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
    lib.lds_fill.restype = ctypes.c_int
    lib.lds_peek.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.lds_peek.restype = ctypes.c_int
    return lib


def _fill(helper, dev, pattern):
    rc = helper.lds_fill(pattern, FILL_BLOCKS, torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0, "lds_fill: hip error %d" % rc


def _same(a, b):
    if isinstance(a, (tuple, list)):
        return all(_same(u, v) for u, v in zip(a, b))
    if a is None:
        return b is None
    return a.dtype == b.dtype and a.shape == b.shape and torch.equal(a.view(-1).view(torch.uint8),
                                                                      b.view(-1).view(torch.uint8))


def _clone(r):
    if isinstance(r, (tuple, list)):
        return tuple(_clone(u) for u in r)
    return None if r is None else r.clone()


def _check(helper, dev, fn, what):
    ref = _clone(fn())
    torch.cuda.synchronize()
    for p in PATTERNS:
        _fill(helper, dev, p)
        got = fn()
        torch.cuda.synchronize()
        assert _same(got, ref), "%s: result changed after LDS filled with 0x%08X" % (what, p)


def test_fill_reaches_the_next_dispatch(dev, helper):
    """The fill pattern is what a later dispatch finds in LDS (on most workgroups)."""
    blocks = 512
    out = torch.empty(blocks * PEEK_WORDS, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    for p in (0x5A5A5A5A, 0x7FC07FC0):
        _fill(helper, dev, p)
        assert helper.lds_peek(out.data_ptr(), blocks, PEEK_WORDS, s) == 0
        torch.cuda.synchronize()
        seen = out.view(blocks, PEEK_WORDS) == (p - (1 << 32) if p >= (1 << 31) else p)
        whole = seen.all(dim=1).float().mean().item()
        assert whole >= 0.5, "only %.3f of the workgroups found pattern 0x%08X" % (whole, p)


def _quantized(q, dev, n, k, gs, bits, dtype, seed):
    return q.quantize(synth.normal_weight(n, k, 1.0, seed=seed).to(dev), gs, bits, dtype)


DECODE_CASES = [
    # (bits, gs, k, n, rows, dtype): kernel path reached
    (4, 64, 1024, 65000, 1, "bf16"),    # streaming, one row tile
    (4, 64, 1024, 65000, 32, "bf16"),   # streaming, two row tiles
    (3, 32, 640, 65000, 16, "fp16"),    # streaming, generic width
    (4, 64, 1024, 20000, 32, "bf16"),   # parts, 2 per row
    (4, 64, 1024, 3001, 32, "bf16"),    # parts (few weight rows)
    (4, 64, 2048, 1000, 8, "bf16"),     # parts
    (8, 64, 1024, 1000, 32, "fp16"),    # parts, 8-bit
    (4, 128, 8192, 500, 16, "bf16"),    # chunked (activations beyond LDS)
    (4, 32, 4096, 600, 32, "bf16"),     # two 16-row blocks
    (2, 32, 640, 1000, 16, "fp16"),
    (3, 32, 640, 1000, 16, "fp16"),
    (5, 32, 640, 1000, 1, "fp16"),
    (6, 32, 640, 1000, 1, "fp16"),
    (6, 32, 640, 1000, 32, "fp16"),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_ignores_stale_lds(dev, helper, case):
    import bit_affine_quantized_qmv_amd as q
    bits, gs, k, n, rows, dtype = DECODE_CASES[case]
    qw = _quantized(q, dev, n, k, gs, bits, dtype, seed=90 + case)
    x = synth.normal_x((rows, k), dtype, seed=91 + case).to(dev)
    _check(helper, dev, lambda: q.qmv(x, qw), DECODE_CASES[case])


def test_argmax_and_gather_ignore_stale_lds(dev, helper):
    import bit_affine_quantized_qmv_amd as q
    qw = _quantized(q, dev, 3001, 1024, 64, 4, "bf16", seed=120)
    x = synth.normal_x((32, 1024), "bf16", seed=121).to(dev)
    ws = q.argmax_workspace(32, dev)
    _check(helper, dev, lambda: q.qmv_argmax(x, qw, workspace=ws), "qmv_argmax")
    ex = q.ExpertWeights.stack([_quantized(q, dev, 700, 1408, 32, 8, "bf16", seed=122 + e) for e in range(4)])
    xg = synth.normal_x((6, 1408), "bf16", seed=126).to(dev)
    idx = torch.tensor([3, 0, 2, 2, 1, 0], dtype=torch.int32, device=dev)
    _check(helper, dev, lambda: q.gather_qmv(xg, ex, idx), "gather_qmv")


@pytest.mark.parametrize("bits", [4, 3])
def test_prefill_ignores_stale_lds(dev, helper, bits):
    """Both prefill kernels: direct-load (4-bit) and register-staged (3-bit)."""
    import bit_affine_quantized_qmv_amd as q
    qw = _quantized(q, dev, 300, 512, 64, bits, "bf16", seed=130 + bits)
    x = synth.normal_x((70, 512), "bf16", seed=131).to(dev)
    _check(helper, dev, lambda: q.qmm_t(x, qw), "qmm_t %d-bit" % bits)


@pytest.mark.parametrize("split", [True, False])
def test_topk_ignores_stale_lds(dev, helper, split):
    import bit_affine_quantized_qmv_amd as q
    logits = synth.normal_x((4, 20000), "bf16", seed=140).to(dev)
    ws = q.topk_workspace(4, dev) if split else None
    _check(helper, dev, lambda: q.topk(logits, 50, workspace=ws, split=split), "topk split=%s" % split)
