"""Pins for the oracle's dequantization (O4), reference product (O5), row gathering (O7)
and acceptance bound (O6)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth


def _random_quantized(seed, n, k, bits, gs, dtype):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32)
    return O.quantize(w, gs, bits, dtype)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_dequant_and_product_against_exact_rationals(bits, gs, dtype):
    """Brute force with fractions.Fraction on tiny shapes: w~ is exact and y_ref lies
    within K * 2^-52 * sum|x w~| of the exact rational sum."""
    n, k, m = 3, 128, 2
    q = _random_quantized(bits * 7 + gs, n, k, bits, gs, dtype)
    rng = np.random.default_rng(gs + bits)
    x_bits = O.to_dtype_bits(rng.standard_normal((m, k)).astype(np.float32), dtype)
    x = O.from_dtype_bits(x_bits, dtype)
    w_deq = O.dequant(q["codes"], q["scales_bits"], q["biases_bits"], gs, dtype)
    y_ref = O.matmul_rows(x, w_deq)
    s = O.from_dtype_bits(q["scales_bits"], dtype)
    b = O.from_dtype_bits(q["biases_bits"], dtype)
    for r in range(m):
        for i in range(n):
            total = Fraction(0)
            mag = Fraction(0)
            for kk in range(k):
                grp = kk // gs
                wv = Fraction(float(s[i, grp])) * int(q["codes"][i, kk]) + Fraction(float(b[i, grp]))
                assert Fraction(float(w_deq[i, kk])) == wv
                term = Fraction(float(x[r, kk])) * wv
                total += term
                mag += abs(term)
            assert abs(Fraction(float(y_ref[r, i])) - total) <= k * Fraction(2) ** -52 * mag


def test_integer_textbook_case():
    """s~ = 1, b~ = 0 and integer x: y is the integer matmul x @ q^T (numpy int64)."""
    rng = np.random.default_rng(3)
    n, k, gs = 5, 256, 64
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    ones = O.to_dtype_bits(np.ones((n, k // gs), dtype=np.float32), "bf16")
    zeros = O.to_dtype_bits(np.zeros((n, k // gs), dtype=np.float32), "bf16")
    x = rng.integers(-8, 9, size=(3, k))
    w_deq = O.dequant(O.unpack(O.pack(codes, 8), 8, k), ones, zeros, gs, "bf16")
    y = O.matmul_rows(x.astype(np.float64), w_deq)
    assert np.array_equal(y, (x @ codes.astype(np.int64).T).astype(np.float64))


def test_closed_form_all_ones_input():
    """x = 1 everywhere: y[n] = sum_g (s~_g * sum_{k in g} q + gs * b~_g)."""
    n, k, gs, bits = 4, 256, 32, 5
    q = _random_quantized(11, n, k, bits, gs, "fp16")
    w_deq = O.dequant(q["codes"], q["scales_bits"], q["biases_bits"], gs, "fp16")
    y = O.matmul_rows(np.ones((1, k)), w_deq)[0]
    s = O.from_dtype_bits(q["scales_bits"], "fp16")
    b = O.from_dtype_bits(q["biases_bits"], "fp16")
    qs = q["codes"].reshape(n, k // gs, gs).sum(axis=2)
    want = (s * qs + gs * b).sum(axis=1)
    assert np.allclose(y, want, rtol=1e-13, atol=0)


def test_product_is_not_transposed_or_bias_free():
    """A non-square case where x @ W~ (transposed) would not even conform, and a bias-free
    product differs: guards against the two plausible slips in O5 / O4."""
    n, k = 3, 64
    q = _random_quantized(5, n, k, 4, 32, "bf16")
    w_deq = O.dequant(q["codes"], q["scales_bits"], q["biases_bits"], 32, "bf16")
    x = np.arange(k, dtype=np.float64)[None, :] / k
    y = O.matmul_rows(x, w_deq)
    assert y.shape == (1, n)
    no_bias = O.dequant(q["codes"], q["scales_bits"], np.zeros_like(q["biases_bits"]), 32, "bf16")
    assert not np.allclose(y, O.matmul_rows(x, no_bias))
    for i in range(n):
        assert y[0, i] == pytest.approx(float(sum(x[0, kk] * w_deq[i, kk] for kk in range(k))), rel=1e-14)


@pytest.mark.parametrize("layout", [
    ((2, 4, 5, 8), (480, 40, 8, 1), 0),        # candle-bmm: heads narrowed out of qkv
    ((2, 2, 3, 5), (60, 15, 5, 1), 0),         # candle-bmm: Linear on a narrowed 4D input
    ((2, 2, 2, 3, 4), (48, 24, 12, 4, 1), 0),  # candle-bmm: rank-5 contiguous
    ((4, 3, 16), (16, 0, 1), 7),               # broadcast rows (stride 0), non-zero offset
    ((3, 1, 16), (64, 16, 1), 5),
])
def test_gather_rows_matches_as_strided(layout):
    shape, stride, offset = layout
    flat = np.arange(1000, dtype=np.float64)
    view = np.lib.stride_tricks.as_strided(flat[offset:], shape=shape,
                                           strides=[s * 8 for s in stride])
    assert np.array_equal(O.gather_rows(flat, shape, stride, offset), view.reshape(-1, shape[-1]))


def test_batch_invariance_by_construction():
    """Row i of a [B,1,K] call is bit-identical to the [1,K] call on that row."""
    q = _random_quantized(9, 16, 256, 4, 64, "bf16")
    w_deq = O.dequant(q["codes"], q["scales_bits"], q["biases_bits"], 64, "bf16")
    x = synth.normal_x((8, 1, 256), "bf16", 3).float().double().numpy()
    flat = x.reshape(-1)
    rows = O.gather_rows(flat, (8, 1, 256), (256, 256, 1))
    y_all = O.matmul_rows(rows, w_deq)
    for i in range(8):
        y_one = O.matmul_rows(O.gather_rows(flat, (1, 256), (256, 1), i * 256), w_deq)
        assert np.array_equal(y_all[i], y_one[0])


def test_ulp_fixtures(golden_dir):
    with open(os.path.join(golden_dir, "float_formats.json")) as f:
        fixtures = json.load(f)
    for case in fixtures["ulp"]:
        assert float(O.ulp(case["v"], case["dtype"])) == case["ulp"], case


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_bound_accepts_correct_rounding_and_rejects_one_step_off(dtype):
    rng = np.random.default_rng(1)
    y_ref = rng.standard_normal(1000) * 10
    y = O.from_dtype_bits(O.to_dtype_bits(y_ref.astype(np.float32), dtype), dtype)
    half_ulp = 0.5 * O.ulp(y_ref, dtype)
    assert np.all(np.abs(y - y_ref) <= half_ulp * (1 + 1e-12))
    off = y + 2 * O.ulp(y, dtype)
    assert np.all(np.abs(off - y_ref) > half_ulp)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_running_sum_closed_form_and_negative_control(dtype, gs):
    """Alternating 2048, 1 inputs ([mlx-4516], first commit: a running sum that half
    precision cannot hold).  Closed form: sum(x) = 2049*K/2 and per group 2049*gs/2.
    On the constructed zero rows y_ref is exactly 0; a kernel that sums x in the input
    dtype in chunks before widening (the defect the page fixes) must fail the bound."""
    k, n, bits = 4096, 6, 5
    x = synth.alternating_x(k, dtype).float().double().numpy()
    assert x.sum() == 2049 * k / 2
    assert x[0, :gs].sum() == 2049 * gs / 2
    c = synth.odd_n_weight(n, k, bits, gs, seed=gs)
    s_bits = O.to_dtype_bits(c["scale_values"], dtype)
    b_bits = O.to_dtype_bits(c["bias_values"], dtype)
    assert np.array_equal(O.from_dtype_bits(b_bits, dtype), c["bias_values"])
    w_deq = O.dequant(c["codes"], s_bits, b_bits, gs, dtype)
    assert np.all(w_deq[c["zero_rows"]] == 0)
    y_ref = O.matmul_rows(x, w_deq)
    assert np.all(y_ref[0, c["zero_rows"]] == 0)
    tol = O.bound(x, w_deq, y_ref, dtype)

    # emulate the defect: chunks of 8 inputs summed in the input dtype, then widened
    x_half = O.to_dtype_bits(x.astype(np.float32), dtype)
    sums = np.zeros(k // gs)
    for g in range(k // gs):
        for c0 in range(g * gs, (g + 1) * gs, 8):
            acc = np.zeros(1, dtype=np.float32)
            for kk in range(c0, c0 + 8):
                acc = O.from_dtype_bits(O.to_dtype_bits(
                    (acc + O.from_dtype_bits(x_half[0, kk:kk + 1], dtype)).astype(np.float32), dtype), dtype)
            sums[g] += acc[0]
    assert sums.sum() == 2048 * k / 2           # every 1.0 was dropped
    s = O.from_dtype_bits(s_bits, dtype)
    b = O.from_dtype_bits(b_bits, dtype)
    sq = (x[0] * c["codes"].astype(np.float64)).reshape(n, k // gs, gs).sum(axis=2)
    y_bug = (s * sq + b * sums[None, :]).sum(axis=1)
    res = O.check(y_bug[None, :], y_ref, tol)
    assert not res["ok"]
    assert set(np.where(c["zero_rows"])[0]) <= {j for _, j in np.argwhere(np.abs(y_bug[None, :] - y_ref) > tol)}
    # and the exact factored form (fp32 widening) passes
    exact_sums = x[0].reshape(k // gs, gs).sum(axis=1)
    y_ok = (s * sq + b * exact_sums[None, :]).sum(axis=1)
    assert O.check(y_ok[None, :], y_ref, tol)["ok"]


def test_probe_page_metric_band(golden_dir):
    """A correct bf16 result on the issue-47331 probe lands in the page's printed band."""
    with open(os.path.join(golden_dir, "probe_band.json")) as f:
        band = json.load(f)["band"]
    w = synth.probe_weight().numpy()
    q = O.quantize(w, 64, 4, "bf16")
    k = 2048
    x = synth.normal_x((2, k), "bf16", 1).float().double().numpy()
    w_deq = O.dequant(q["codes"], q["scales_bits"], q["biases_bits"], 64, "bf16")
    y = O.matmul_rows(x, w_deq)
    y_bf16 = O.bf16_bits_to_f64(O.f32_to_bf16_bits(y.astype(np.float32)))
    g = np.arange(k) // 64
    ref = x @ (q["s32"][:, g].astype(np.float64) * q["codes"] + q["b32"][:, g]).T
    metric = O.page_metric(y_bf16, ref)
    assert np.all((metric > band[0]) & (metric < band[1])), metric
