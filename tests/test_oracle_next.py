"""Pins of the oracle functions behind the rows that extend the hot path (gathered weights,
...), checked against independent computations."""
import numpy as np

import oracle as O


def _int_expert(rng, n, k, bits):
    codes = rng.integers(0, 2 ** bits, size=(n, k))
    g = k // 32
    ones = np.full((n, g), O.to_dtype_bits(np.float32(1.0), "bf16"), dtype=np.uint16)
    zeros = np.zeros((n, g), dtype=np.uint16)
    return codes, (O.pack(codes, bits), ones, zeros)


def test_gather_integer_textbook():
    # s = 1, b = 0, integer x: row r is an exact integer product with expert index[r]'s codes
    rng = np.random.default_rng(7)
    n, k, bits, e = 5, 64, 3, 4
    made = [_int_expert(rng, n, k, bits) for _ in range(e)]
    codes = np.stack([c for c, _ in made])            # [E, N, K]
    x = rng.integers(-4, 5, size=(6, k))
    idx = np.array([2, 0, 3, 3, 1, 2])
    ref = O.gather_reference(x.astype(np.float64), [t for _, t in made], idx, k, 32, bits, "bf16")
    expect = np.einsum("rk,rnk->rn", x, codes[idx])   # gathered integer products
    assert np.array_equal(ref["y_ref"], expect.astype(np.float64))


def test_gather_single_expert_is_plain_reference():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((7, 128)).astype(np.float32)
    qz = O.quantize(w, 64, 4, "fp16")
    t = (O.pack(qz["codes"], 4), qz["scales_bits"], qz["biases_bits"])
    x = rng.standard_normal((3, 128))
    g = O.gather_reference(x, [t], np.zeros(3, dtype=np.int64), 128, 64, 4, "fp16")
    plain = O.reference(x, *t, 128, 64, 4, "fp16")
    assert np.array_equal(g["y_ref"], plain["y_ref"])
    assert np.allclose(g["tol"], plain["tol"], rtol=1e-12, atol=0)   # a bound, summed row by row


def test_gather_out_of_range_rows_are_nan():
    rng = np.random.default_rng(9)
    _, t = _int_expert(rng, 4, 32, 2)
    x = np.ones((3, 32))
    g = O.gather_reference(x, [t, t], np.array([-1, 1, 2]), 32, 32, 2, "bf16")
    assert np.isnan(g["y_ref"][0]).all() and np.isnan(g["y_ref"][2]).all()
    assert np.isfinite(g["y_ref"][1]).all()


def test_dequantize_dtype_on_grid_is_exact():
    # power-of-two scales, on-grid biases: every dequantized value is exact in both dtypes
    rng = np.random.default_rng(10)
    for dtype in ("bf16", "fp16"):
        codes = rng.integers(0, 16, size=(3, 64))
        s = np.array([[2.0 ** -6, 2.0 ** -3]] * 3)
        b = np.array([[-0.25, 0.5]] * 3)
        got = O.from_dtype_bits(O.dequantize_dtype(codes, O.to_dtype_bits(s, dtype), O.to_dtype_bits(b, dtype),
                                                   32, dtype), dtype)
        expect = codes * np.repeat(s, 32, axis=1) + np.repeat(b, 32, axis=1)
        assert np.array_equal(got, expect)


def test_dequantize_dtype_within_rounding_of_exact():
    # against the exact float64 dequantization: at most half a float32 step plus half a
    # dtype step away (two roundings)
    rng = np.random.default_rng(11)
    w = rng.standard_normal((6, 256)).astype(np.float32)
    for dtype in ("bf16", "fp16"):
        qz = O.quantize(w, 64, 5, dtype)
        exact = O.dequant(qz["codes"], qz["scales_bits"], qz["biases_bits"], 64, dtype)
        got = O.from_dtype_bits(O.dequantize_dtype(qz["codes"], qz["scales_bits"], qz["biases_bits"], 64, dtype),
                                dtype)
        f32_half = np.abs(exact) * 2.0 ** -24
        assert np.all(np.abs(got - exact) <= 0.5 * O.ulp(exact, dtype) + f32_half + 1e-300)


def test_embedding_integer_rows():
    rng = np.random.default_rng(12)
    codes, t = _int_expert(rng, 9, 64, 4)
    rows = O.embedding_reference(*t, [4, 0, 8, 4, 9, -2], 64, 32, 4, "bf16")
    assert rows[4] is None and rows[5] is None
    for r, i in zip(rows[:4], [4, 0, 8, 4]):
        assert np.array_equal(O.from_dtype_bits(r, "bf16"), codes[i].astype(np.float64))


def test_argmax_acceptable_exact_and_ties():
    # exact integer logits (tolerance 0): the unique maximum, or every tied maximum
    y = np.array([[1.0, 5.0, 3.0, 5.0], [-2.0, -1.0, -3.0, -1.5]])
    got = O.argmax_acceptable(y, np.zeros_like(y))
    assert got == [{1, 3}, {1}]
    # tolerance widens the set to the values that could overtake the maximum
    got = O.argmax_acceptable(y, np.full_like(y, 0.3))
    assert got == [{1, 3}, {1, 3}]


def _bits(vals, dtype="bf16"):
    return O.to_dtype_bits(np.asarray(vals, dtype=np.float32), dtype)


def test_topk_matches_descending_sort():
    # distinct values: the order is the plain descending sort
    rng = np.random.default_rng(7)
    v = rng.permutation(np.arange(-40, 40, dtype=np.float32))[None, :] * 0.25
    for dtype in ("bf16", "fp16"):
        idx, val = O.topk_rows(_bits(v, dtype), 9, dtype)
        want = np.argsort(-v[0], kind="stable")[:9]
        assert idx[0].tolist() == want.tolist()
        assert val[0].tolist() == sorted(v[0].tolist(), reverse=True)[:9]


def test_topk_ties_take_lower_columns_first():
    idx, val = O.topk_rows(_bits([[1.0, 3.0, 3.0, 2.0, 3.0, 2.0]]), 4, "bf16")
    assert idx[0].tolist() == [1, 2, 4, 3]
    assert val[0].tolist() == [3.0, 3.0, 3.0, 2.0]


def test_topk_nan_infinities_and_signed_zero():
    row = np.array([[0.0, -0.0, np.nan, np.inf, -np.inf, 1.0, -2.0]], dtype=np.float16)
    idx, val = O.topk_rows(row.view(np.uint16), 7, "fp16")   # exact fp16 patterns
    assert idx[0].tolist() == [2, 3, 5, 0, 1, 6, 4]
    assert np.isnan(val[0, 0]) and val[0, 1] == np.inf and val[0, -1] == -np.inf
    assert not np.signbit(val[0, 3]) and np.signbit(val[0, 4])


def test_topk_k1_is_first_maximal_column():
    rng = np.random.default_rng(3)
    v = rng.integers(-3, 4, size=(6, 40)).astype(np.float32)   # many ties
    idx, val = O.topk_rows(_bits(v), 1, "bf16")
    for r in range(6):
        assert idx[r, 0] == int(np.argmax(v[r])) and val[r, 0] == v[r].max()


def test_topk_full_k_is_a_permutation():
    rng = np.random.default_rng(5)
    v = rng.integers(-5, 5, size=(3, 33)).astype(np.float32)
    idx, val = O.topk_rows(_bits(v), 33, "bf16")
    for r in range(3):
        assert sorted(idx[r].tolist()) == list(range(33))
        assert all(val[r, j] >= val[r, j + 1] for j in range(32))
