"""Pins for the oracle's per-group min/max quantizer (O1) and its storage casts."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

CASES = [(b, gs, dt) for b in (2, 3, 4, 5, 6, 8) for gs in (32, 64, 128) for dt in ("bf16", "fp16")]


def _weights(seed, kind, n=6, k=256):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((n, k)).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(-3, 5, (n, k)).astype(np.float32)
    return (rng.standard_t(2, (n, k)) * 0.1).astype(np.float32)        # heavy tails


@pytest.mark.parametrize("bits,gs,dtype", CASES)
def test_round_trip_within_half_step(bits, gs, dtype):
    """|w - (s32*q + b32)| <= s32/2 (+ 2 float32 ulps of w - b32 for the two rounded ops)."""
    for kind in ("normal", "uniform", "heavy"):
        w = _weights(bits * 1000 + gs, kind)
        q = O.quantize(w, gs, bits, dtype)
        codes = q["codes"].astype(np.float64)
        g = np.arange(w.shape[1]) // gs
        s = q["s32"][:, g].astype(np.float64)
        b = q["b32"][:, g].astype(np.float64)
        err = np.abs(w.astype(np.float64) - (s * codes + b))
        slack = 2.0 * np.spacing(np.abs(w - q["b32"][:, g]).astype(np.float32)).astype(np.float64)
        assert np.all(err <= s / 2 + slack), (kind, float((err - s / 2 - slack).max()))
        assert codes.min() >= 0 and codes.max() <= 2 ** bits - 1


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_on_grid_recovers_codes_scale_and_bias(bits):
    """W = b + s*j with s a power of two and both 0 and 2^bits-1 in every group: every
    group must come back exactly, with its own (s, b) (catches a wrong divisor, a wrong
    bias, or a wrong row/group indexing)."""
    rng = np.random.default_rng(bits)
    n, k, gs = 4, 256, 64
    qmax = 2 ** bits - 1
    j = rng.integers(0, qmax + 1, size=(n, k))
    j[:, ::gs] = 0
    j[:, 1::gs] = qmax
    s = 2.0 ** rng.integers(-8, 0, size=(n, k // gs))
    b = rng.integers(-64, 64, size=(n, k // gs)) * 2.0 ** -5
    w = (np.repeat(b, gs, axis=1) + np.repeat(s, gs, axis=1) * j).astype(np.float32)
    q = O.quantize(w, gs, bits, "bf16")
    assert np.array_equal(q["codes"], j)
    assert np.array_equal(q["s32"], s.astype(np.float32))
    assert np.array_equal(q["b32"], b.astype(np.float32))


def test_constant_group_gets_code_zero():
    w = np.full((2, 64), 0.37, dtype=np.float32)
    w[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q = O.quantize(w, 32, 4, "fp16")
    assert np.all(q["codes"][0] == 0) and np.all(q["codes"][1, :32] == 0)
    assert q["s32"][0, 0] == 0 and q["b32"][0, 0] == np.float32(0.37)
    assert q["codes"][1, 32:].max() == 15


def test_rounds_half_to_even():
    """(w - b)/s exactly halfway between codes rounds to the even code."""
    gs = 32
    w = np.zeros((1, gs), dtype=np.float32)
    w[0, 1] = 15.0           # s = 1, b = 0 for 4 bits
    w[0, 2] = 2.5            # -> 2
    w[0, 3] = 3.5            # -> 4
    q = O.quantize(w, gs, 4, "bf16")
    assert q["s32"][0, 0] == 1.0
    assert q["codes"][0, 2] == 2 and q["codes"][0, 3] == 4


def test_storage_casts_match_torch_and_formats(golden_dir):
    with open(os.path.join(golden_dir, "float_formats.json")) as f:
        fixtures = json.load(f)
    for case in fixtures["bf16_rne"]:
        got = int(O.f32_to_bf16_bits(np.array([case["f32"]], dtype=np.float32))[0])
        assert got == int(case["bits"], 16), case
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    t = torch.from_numpy(a)
    assert np.array_equal(O.f32_to_bf16_bits(a), t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    a16 = a[np.abs(a) < 60000]
    t16 = torch.from_numpy(a16).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_f16_bits(a16), t16)
    bits = O.f32_to_bf16_bits(a)
    assert np.array_equal(O.bf16_bits_to_f64(bits), t.to(torch.bfloat16).double().numpy())


def test_scales_and_biases_are_rne_casts_of_fp32_parameters():
    w = _weights(7, "normal")
    for dt in ("bf16", "fp16"):
        q = O.quantize(w, 64, 4, dt)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float16
        s_t = torch.from_numpy(q["s32"]).to(tdt).double().numpy()
        b_t = torch.from_numpy(q["b32"]).to(tdt).double().numpy()
        assert np.array_equal(O.from_dtype_bits(q["scales_bits"], dt), s_t)
        assert np.array_equal(O.from_dtype_bits(q["biases_bits"], dt), b_t)
