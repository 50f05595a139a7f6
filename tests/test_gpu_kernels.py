"""GPU parity of the HIP path against the CPU oracle at small sizes (several tiles, ragged
tails, every codec width).  All calls go through the C ABI (libqmm.so)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from qmm_testlib import (TORCH_DTYPE, assert_close, gather, half_bits, oracle_view_of,
                         reference_rows, require_gpu, upload_oracle_weight, values, words)

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 8]
GS = [32, 64, 128]
DT = ["bf16", "fp16"]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _rand_w(n, k, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((n, k)).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(-2, 3, (n, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    w[:, :32] = 0.5                                     # a constant group
    return w


# ---------------------------------------------------------------- qmm_quantize
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dtype", DT)
def test_quantize_bit_exact(dev, bits, gs, dtype):
    import bit_affine_quantized_qmv_amd as q
    for kind in ("normal", "uniform", "const"):
        w = _rand_w(37, 384, bits * 100 + gs, kind)
        qw = q.quantize(torch.from_numpy(w).to(dev), gs, bits, dtype)
        torch.cuda.synchronize()
        ref = O.quantize(w, gs, bits, dtype)
        assert np.array_equal(words(qw.w_packed), O.pack(ref["codes"], bits)), kind
        assert np.array_equal(half_bits(qw.scales), ref["scales_bits"]), kind
        assert np.array_equal(half_bits(qw.biases), ref["biases_bits"]), kind


def test_quantize_strided_rows(dev):
    import bit_affine_quantized_qmv_amd as q
    w = _rand_w(20, 512, 5)
    buf = torch.zeros(20, 640)
    buf[:, :512] = torch.from_numpy(w)
    qw = q.quantize(buf.to(dev)[:, :512], 64, 4, "bf16")
    ref = O.quantize(w, 64, 4, "bf16")
    assert np.array_equal(words(qw.w_packed), O.pack(ref["codes"], 4))


@pytest.mark.parametrize("bits", [3, 5, 6, 8])
def test_quantize_unaligned_stride_and_short_rows(dev, bits):
    """Rows 4-byte but not 16-byte aligned (stride 517 floats: element-wise loads) and rows
    that end inside a 256-element segment (K = 96 and 352, group 32), bit-exact."""
    import bit_affine_quantized_qmv_amd as q
    for k in (96, 352):
        w = _rand_w(11, k, 40 + bits + k)
        buf = torch.zeros(11, 517)
        buf[:, :k] = torch.from_numpy(w)
        qw = q.quantize(buf.to(dev)[:, :k], 32, bits, "fp16")
        torch.cuda.synchronize()
        ref = O.quantize(w, 32, bits, "fp16")
        assert np.array_equal(words(qw.w_packed), O.pack(ref["codes"], bits)), k
        assert np.array_equal(half_bits(qw.scales), ref["scales_bits"]), k
        assert np.array_equal(half_bits(qw.biases), ref["biases_bits"]), k


# ---------------------------------------------------------------- unpack probes
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dtype", DT)
def test_one_hot_unpack(dev, bits, gs, dtype):
    """s~ = 1, b~ = 0 and x = e_k: y[n] = q[n, k] exactly, for every k of a 128-k slice
    (32 one-hot rows per decode call), and through the prefill kernel (128 rows)."""
    import bit_affine_quantized_qmv_amd as q
    rng = np.random.default_rng(bits + gs)
    n, k = 45, 256
    codes = rng.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)
    ones = O.to_dtype_bits(np.ones((n, k // gs), np.float32), dtype)
    zeros = O.to_dtype_bits(np.zeros((n, k // gs), np.float32), dtype)
    qw = upload_oracle_weight({"codes": codes, "scales_bits": ones, "biases_bits": zeros,
                               "bits": bits, "group_size": gs, "dtype": dtype}, dev)
    eye = torch.eye(k, dtype=TORCH_DTYPE[dtype], device=dev)
    for k0 in range(0, k, 32):
        y = q.qmv(eye[k0:k0 + 32], qw)
        assert np.array_equal(values(y), codes[:, k0:k0 + 32].T.astype(np.float64)), k0
    y = q.qmm_t(eye, qw)
    assert np.array_equal(values(y), codes.T.astype(np.float64))


# ---------------------------------------------------------------- decode family
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dtype", DT)
def test_decode_parity_ragged(dev, bits, gs, dtype):
    import bit_affine_quantized_qmv_amd as q
    n, k = 1000, 640                         # N not a multiple of 16 or of any tile
    w = _rand_w(n, k, bits * 7 + gs)
    qo = O.quantize(w, gs, bits, dtype)
    qw = upload_oracle_weight(qo, dev)
    for m in (1, 3, 16, 17, 32):
        x = synth.normal_x((m, k), dtype, seed=m).to(dev)
        y = q.qmv(x, qw)
        assert_close(y, reference_rows(values(x), qw, dtype), "m=%d" % m)


def test_decode_wide_tiles(dev):
    """N large enough for the 4-tile-per-wave launch, with a ragged tail."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 40000 + 37, 256
    for bits, gs in ((4, 64), (8, 32), (3, 128)):
        w = synth.normal_weight(n, k, 0.02, seed=bits).numpy()
        qw = q.quantize(torch.from_numpy(w).to(dev), gs, bits, "bf16")
        rows = synth.rows_sample(n, 300, seed=bits)
        for m in (1, 32):
            x = synth.normal_x((m, k), "bf16", seed=m).to(dev)
            y = q.qmv(x, qw)
            ref = reference_rows(values(x), qw, "bf16", rows=rows)
            assert_close(y[:, rows], ref, "bits=%d m=%d" % (bits, m))


def test_decode_k_chunks(dev):
    """K larger than one LDS activation chunk (2048 at <= 16 rows, 1024 at <= 32 rows)."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 300, 4096 + 1024
    for bits, gs in ((4, 128), (8, 64), (5, 32)):
        w = _rand_w(n, k, bits)
        qw = upload_oracle_weight(O.quantize(w, gs, bits, "fp16"), dev)
        for m in (5, 29):
            x = synth.normal_x((m, k), "fp16", seed=m).to(dev)
            assert_close(q.qmv(x, qw), reference_rows(values(x), qw, "fp16"), "bits=%d m=%d" % (bits, m))


def test_batch_invariance_and_strided_rows(dev):
    """Row i of every [B,1,K] call equals the [1,K] call on row i bit for bit; rows read
    through a stride (every other row of a [2B,K] buffer) equal the dense call; forcing
    one grid slice per batch element changes nothing."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 777, 1024
    for bits in (4, 8, 6):
        qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=bits).to(dev), 64, bits, "bf16")
        x32 = synth.normal_x((32, 1, k), "bf16", seed=bits).to(dev)
        singles = [q.qmv(x32[i], qw) for i in range(32)]
        for b in (1, 2, 4, 8, 16, 32):
            y = q.qmv(x32[:b], qw)
            for i in range(b):
                assert torch.equal(y[i], singles[i]), (bits, b, i)
        buf = synth.normal_x((64, k), "bf16", seed=99).to(dev)
        y_str = q.qmv(buf[0::2], qw)
        y_den = q.qmv(buf[0::2].contiguous(), qw)
        assert torch.equal(y_str, y_den)
        y_forced = q.qmv(x32, qw, flags=q.QMM_FLAG_FORCE_STRIDED)
        assert torch.equal(y_forced, q.qmv(x32, qw))
        assert_close(y_str, reference_rows(gather(buf, buf[0::2]), qw, "bf16"), "strided")


# ---------------------------------------------------------------- prefill family
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dtype", DT)
def test_prefill_parity_ragged(dev, bits, dtype):
    import bit_affine_quantized_qmv_amd as q
    n, k = 333, 384
    for gs in GS:
        w = _rand_w(n, k, bits * 3 + gs)
        qw = upload_oracle_weight(O.quantize(w, gs, bits, dtype), dev)
        for m in (33, 200):
            x = synth.normal_x((m, k), dtype, seed=m + gs).to(dev)
            assert_close(q.qmm_t(x, qw), reference_rows(values(x), qw, dtype), "gs=%d m=%d" % (gs, m))


def test_prefill_strided_view_matches_contiguous(dev):
    """A view narrowed on the sequence dim (two strided levels) gives the same bits as its
    contiguous copy, at offset 0 and at a non-zero start."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 520, 512
    qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=7).to(dev), 128, 4, "bf16")
    buf = synth.normal_x((3, 100, k), "bf16", seed=8).to(dev)
    for start in (0, 24):
        view = buf[:, start:start + 50, :]
        y = q.qmm_t(view, qw)
        assert torch.equal(y, q.qmm_t(view.contiguous(), qw))
        assert_close(y, reference_rows(gather(buf, view), qw, "bf16"), "start=%d" % start)


def test_qmm_t_small_rows_use_decode_kernels(dev):
    import bit_affine_quantized_qmv_amd as q
    qw = q.quantize(synth.normal_weight(300, 256, 1.0, seed=1).to(dev), 64, 4, "bf16")
    x = synth.normal_x((2, 4, 256), "bf16", seed=2).to(dev)
    assert torch.equal(q.qmm_t(x, qw), q.qmv(x, qw))


# ---------------------------------------------------------------- layouts and edges
def test_candle_layouts(dev):
    """The candle page's layouts (K widened to 128): a 4D view with batch strides that do
    not merge into one, a Linear input narrowed on dim 1, and a rank-5 contiguous input.
    All fold into <= 2 strided levels here and must be computed row by row correctly."""
    import bit_affine_quantized_qmv_amd as q
    k = 128
    qw = q.quantize(synth.normal_weight(70, k, 1.0, seed=3).to(dev), 32, 4, "fp16")
    qkv = synth.normal_x((2, 12, 5, k), "fp16", seed=4).to(dev)
    lin = synth.normal_x((2, 4, 3, k), "fp16", seed=5).to(dev)
    r5 = synth.normal_x((2, 2, 2, 3, k), "fp16", seed=6).to(dev)
    for buf, view in ((qkv, qkv[:, 0:4]), (lin, lin[:, 0:2]), (r5, r5)):
        y = q.qmm_t(view, qw)
        assert_close(y, reference_rows(gather(buf, view), qw, "fp16"), str(tuple(view.shape)))
        assert torch.equal(y, q.qmm_t(view.contiguous(), qw))


def test_three_level_layout_rejected_untouched(dev):
    import bit_affine_quantized_qmv_amd as q
    k = 128
    qw = q.quantize(synth.normal_weight(16, k, 1.0, seed=3).to(dev), 32, 4, "bf16")
    buf = synth.normal_x((2, 3, 4, 5, k), "bf16", seed=1).to(dev)
    view = buf[:, 0:2, 0:3, 0:4]                 # three non-mergeable levels
    y = torch.full((2, 2, 3, 4, 16), float("nan"), dtype=torch.bfloat16, device=dev)
    with pytest.raises(q.QmmError) as e:
        q.qmm_t(view, qw, out=y)
    assert e.value.code == -4
    assert torch.isnan(y).all()


def test_every_output_written_and_no_spill(dev):
    """NaN-poisoned output fully overwritten; guard bands on both sides stay untouched."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 203, 256
    qw = q.quantize(synth.normal_weight(n, k, 1.0, seed=9).to(dev), 64, 5, "bf16")
    for m in (1, 7, 32, 45):
        guard = 4096
        raw = torch.full((guard * 2 + m * n,), 12345.0, dtype=torch.bfloat16, device=dev)
        y = raw[guard:guard + m * n].view(m, n)
        y.fill_(float("nan"))
        x = synth.normal_x((m, k), "bf16", seed=m).to(dev)
        q.qmm_t(x, qw, out=y)
        assert not torch.isnan(y).any(), m
        assert (raw[:guard] == 12345.0).all() and (raw[guard + m * n:] == 12345.0).all(), m


def test_empty_and_errors(dev):
    import bit_affine_quantized_qmv_amd as q
    qw = q.quantize(synth.normal_weight(16, 128, 1.0, seed=3).to(dev), 32, 4, "bf16")
    y = q.qmm_t(torch.empty(0, 128, dtype=torch.bfloat16, device=dev), qw)
    assert y.shape == (0, 16)
    with pytest.raises(q.QmmError) as e:
        q.qmv(torch.zeros(33, 128, dtype=torch.bfloat16, device=dev), qw)
    assert e.value.code == -3
    with pytest.raises(q.QmmError):
        q.qmm_t(torch.zeros(4, 128, dtype=torch.float16, device=dev), qw)


def test_large_k_seventeen_to_32_rows(dev):
    """17..32 rows at K = 4096 (activations too large for one LDS block of 32 rows): rows
    equal the single-row calls bit for bit, for one segment, for a two-level layout of
    16-row segments, and with the fused argmax."""
    import bit_affine_quantized_qmv_amd as q
    n, k = 3000, 4096
    qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=41).to(dev), 128, 4, "bf16")
    x = synth.normal_x((32, k), "bf16", seed=42).to(dev)
    singles = torch.cat([q.qmv(x[i:i + 1], qw) for i in range(32)])
    for m in (17, 20, 32):
        assert torch.equal(q.qmv(x[:m], qw), singles[:m]), m
    buf = synth.normal_x((2, 20, k), "bf16", seed=43).to(dev)
    view = buf[:, :16, :]                          # two segments of 16 rows
    y = q.qmv(view, qw)
    for b in range(2):
        for i in (0, 15):
            assert torch.equal(y[b, i], q.qmv(view[b, i:i + 1], qw)[0]), (b, i)
    assert_close(y.reshape(32, n), reference_rows(gather(buf, view), qw, "bf16"), "two segments")
    idx, val, yl = q.qmv_argmax(x[:20], qw)
    assert torch.equal(yl, singles[:20])
    assert torch.equal(idx, torch.argmax(yl.float(), dim=1).to(torch.int32))


def test_concurrent_calls_from_threads(dev):
    """Calls from several host threads, each on its own stream and with its own shape (so
    different launch settings are looked up at once), give the sequential results."""
    import threading
    import bit_affine_quantized_qmv_amd as q
    cases = []
    for i, (k, n, m, bits) in enumerate([(1024, 3000, 32, 4), (2048, 1500, 8, 4), (4096, 700, 1, 8), (1056, 900, 20, 4)]):
        qw = q.quantize(synth.normal_weight(n, k, 0.02, seed=60 + i).to(dev), 32, bits, "bf16")
        x = synth.normal_x((m, k), "bf16", seed=70 + i).to(dev)
        cases.append((qw, x, q.qmv(x, qw)))
    torch.cuda.synchronize()
    outs = [None] * len(cases)
    errors = []

    def work(j):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                qw, x, _ = cases[j]
                ys = [q.qmv(x, qw) for _ in range(20)]
            s.synchronize()
            outs[j] = ys
        except Exception as e:          # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for j, (_, _, ref) in enumerate(cases):
        for y in outs[j]:
            assert torch.equal(y, ref), j
