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
