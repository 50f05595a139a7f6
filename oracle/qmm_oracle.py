"""CPU oracle for affine group-quantized matrix multiplication, y = x . dequant(W)^T.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the tests,
the smoke check and the CPU-baseline leg of the benchmark may call it.  It shares no
code, table or constant generator with the HIP path and never imports it.

Plain, slow and checkable by eye: numpy float32 where the method fixes single-precision
arithmetic (the quantizer), exact float64 / integer arithmetic everywhere else.

Sources (the web pages this method is described on):
  [issue-47331]  "MetalConfig quantization: batched generate silently corrupts all rows
                 after the first" (huggingface/transformers issue 47331), sections
                 "Root cause" (kernel probe, layout table) and "Fix".
  [bits8-report] "Metal Kernel Bits=8 修复最终报告", section 3.1 (4-bit and 8-bit packing
                 formulas).
  [mlx-4516]     ml-explore/mlx pull request 4516, conversation (first commit text:
                 widening every input before the bias * sum(x) term; the running-sum test)
                 and "Correctness" (half a bfloat16 step of a float64 reference).
  [candle-bmm]   candle pitfall page "Metal 上批量 matmul 结果不对", sections 出处 and
                 怎么确认没中招 (batch-stride merge rule).

Readings taken where the pages are silent (each one is listed in the design notes):
  * scale s = (max - min) / (2^bits - 1) and bias = min per (row, group), in fp32;
    codes = round-half-even((w - bias) / s) clamped to [0, 2^bits - 1]; a constant group
    (s == 0) gets code 0.  Scales and biases are cast to the storage dtype (RNE) after the
    codes are computed, as the probe in [issue-47331] casts them after quantizing.
  * 2/3/5/6-bit codes use the same little-endian bitstream that the 4/8-bit formulas of
    [bits8-report] describe: code k of a row sits at bit k*bits of that row's stream,
    spilling into the next uint32 when it straddles a word.
  * y_ref is the exact (float64) sum over k of x * (s~ * q + b~), where s~ and b~ are
    the half-precision values the kernel receives.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
DTYPES = (BF16, FP16)

# mantissa precision p (including the implicit bit) and subnormal spacing per dtype
_PRECISION = {BF16: 8, FP16: 11}
_SUBNORMAL_SPACING = {BF16: 2.0 ** -133, FP16: 2.0 ** -24}

# relative term of the acceptance bound: |y - y_ref| <= REL_TOL * sum|x w~| + 0.5 ulp(y_ref)
REL_TOL = 4e-3


# ----------------------------------------------------------------------------------
# half-precision storage formats, written out by bit manipulation
# ----------------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round half to even); returns uint16 bit patterns.

    bfloat16 is the upper half of a float32; rounding adds 0x7FFF plus the lowest kept
    bit before truncating, which is round-to-nearest with ties to the even pattern.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    assert np.all(np.isfinite(a)), "oracle assumes finite inputs"
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return ((u >> 16) & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_f16_bits(a) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast is round half to even)."""
    a = np.asarray(a, dtype=np.float32)
    assert np.all(np.isfinite(a)), "oracle assumes finite inputs"
    h = a.astype(np.float16)
    assert np.all(np.isfinite(h)), "value overflows float16"
    return h.view(np.uint16)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_dtype_bits(a, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == BF16 else f32_to_f16_bits(a)


def from_dtype_bits(bits, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(bits) if dtype == BF16 else f16_bits_to_f64(bits)


# ----------------------------------------------------------------------------------
# O1: per-group min/max affine quantizer
# ----------------------------------------------------------------------------------
def quantize(w, group_size: int, bits: int, dtype: str) -> dict:
    """Quantize W [N, K] (float32) per row and per group of `group_size` columns.

    The codec is w ~= s * q + b with q in [0, 2^bits - 1] and one (s, b) per (row, group)
    ([issue-47331], kernel probe: quantize, then cast scales/biases to bf16).  All
    arithmetic is float32 with IEEE round-to-nearest-even, one operation at a time:
        s32 = fl(fl(max - min) / (2^bits - 1)),  b32 = min
        q   = clamp(rint(fl(fl(w - b32) / s32)), 0, 2^bits - 1),  q = 0 where s32 == 0
    Returns codes (uint8 [N, K]), s32/b32 (float32 [N, G]) and the storage bit patterns
    of s~ = RNE_dtype(s32), b~ = RNE_dtype(b32) (uint16 [N, G]).
    """
    assert bits in (2, 3, 4, 5, 6, 8) and group_size in (32, 64, 128) and dtype in DTYPES
    w = np.asarray(w, dtype=np.float32)
    n_rows, k_cols = w.shape
    assert k_cols % group_size == 0
    n_groups = k_cols // group_size
    wg = w.reshape(n_rows, n_groups, group_size)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    qmax = np.float32(2 ** bits - 1)
    s32 = (hi - lo) / qmax                      # two float32 operations, each rounded
    b32 = lo
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (wg - b32[:, :, None]) / s32[:, :, None]
    q = np.clip(np.rint(t), np.float32(0), qmax)
    q = np.where(s32[:, :, None] == 0, np.float32(0), q)
    codes = q.astype(np.uint8).reshape(n_rows, k_cols)
    return {
        "codes": codes,
        "s32": s32.astype(np.float32),
        "b32": b32.astype(np.float32),
        "scales_bits": to_dtype_bits(s32, dtype),
        "biases_bits": to_dtype_bits(b32, dtype),
        "group_size": group_size,
        "bits": bits,
        "dtype": dtype,
    }


# ----------------------------------------------------------------------------------
# O2 / O3: little-endian bitstream packing into uint32 words
# ----------------------------------------------------------------------------------
def pack(codes, bits: int) -> np.ndarray:
    """Pack codes [N, K] into uint32 words [N, K*bits/32].

    Code k of a row starts at bit p = k*bits of the row's stream: word p // 32, bit p % 32;
    if it does not fit, its high bits continue at bit 0 of the next word.  For 4 and
    8 bits this is the word index / shift of [bits8-report] section 3.1
    (word = k // (32/bits), shift = (k % (32/bits)) * bits).
    """
    codes = np.asarray(codes)
    n_rows, k_cols = codes.shape
    assert (k_cols * bits) % 32 == 0
    assert codes.size == 0 or int(codes.max()) < (1 << bits)
    words = np.zeros((n_rows, k_cols * bits // 32), dtype=np.uint64)
    q = codes.astype(np.uint64)
    for k in range(k_cols):
        word, shift = divmod(k * bits, 32)
        words[:, word] |= (q[:, k] << np.uint64(shift)) & np.uint64(0xFFFFFFFF)
        if shift + bits > 32:
            words[:, word + 1] |= q[:, k] >> np.uint64(32 - shift)
    return words.astype(np.uint32)


def unpack(words, bits: int, k_cols: int) -> np.ndarray:
    """Inverse of pack(): read code k from bits [k*bits, k*bits + bits) of the row stream."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    n_rows = words.shape[0]
    mask = np.uint64((1 << bits) - 1)
    codes = np.zeros((n_rows, k_cols), dtype=np.uint8)
    for k in range(k_cols):
        word, shift = divmod(k * bits, 32)
        v = words[:, word] >> np.uint64(shift)
        if shift + bits > 32:
            v = v | (words[:, word + 1] << np.uint64(32 - shift))
        codes[:, k] = (v & mask).astype(np.uint8)
    return codes


# ----------------------------------------------------------------------------------
# O4: dequantize, exactly, in float64
# ----------------------------------------------------------------------------------
def dequant(codes, scales_bits, biases_bits, group_size: int, dtype: str) -> np.ndarray:
    """w~[n, k] = s~[n, k // gs] * q[n, k] + b~[n, k // gs] in float64.

    s~ * q needs at most 11 + 8 significant bits, so the product is exact; the sum is
    exact whenever the exponent gap to b~ is below 34 bits (true for every workload used
    here), otherwise within one float64 ulp.
    """
    codes = np.asarray(codes)
    s = from_dtype_bits(scales_bits, dtype)
    b = from_dtype_bits(biases_bits, dtype)
    g_of_k = np.arange(codes.shape[1]) // group_size
    return s[:, g_of_k] * codes.astype(np.float64) + b[:, g_of_k]


# ----------------------------------------------------------------------------------
# O5 / O7: activations from (shape, stride, offset), and the float64 reference product
# ----------------------------------------------------------------------------------
def gather_rows(flat_values, shape, stride, offset: int = 0) -> np.ndarray:
    """Collect every activation row of a strided view as float64 [R, K].

    Row r is the r-th index tuple of shape[:-1] in row-major order; its element k lives
    at flat_values[offset + sum_i idx_i * stride_i + k * stride[-1]].  This walks every
    index explicitly, independently of how a dispatcher might fold the batch dims.
    """
    flat = np.asarray(flat_values, dtype=np.float64).reshape(-1)
    shape = [int(v) for v in shape]
    stride = [int(v) for v in stride]
    k_cols = shape[-1]
    batch = shape[:-1]
    n_rows = int(np.prod(batch)) if batch else 1
    out = np.empty((n_rows, k_cols), dtype=np.float64)
    k_idx = np.arange(k_cols) * stride[-1]
    for r in range(n_rows):
        rem, base = r, offset
        for dim in range(len(batch) - 1, -1, -1):
            rem, i = divmod(rem, batch[dim])
            base += i * stride[dim]
        out[r] = flat[base + k_idx]
    return out


def matmul_rows(x_rows, w_deq) -> np.ndarray:
    """y_ref[r, :] = W~ @ x_r in float64, one activation row at a time.

    Every row goes through the same routine on its own, so a row's reference value does
    not depend on which other rows share the call (batch invariance by construction).
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    w_deq = np.asarray(w_deq, dtype=np.float64)
    y = np.empty((x_rows.shape[0], w_deq.shape[0]), dtype=np.float64)
    for r in range(x_rows.shape[0]):
        y[r] = w_deq @ x_rows[r]
    return y


def abs_products(x_rows, w_deq) -> np.ndarray:
    """sum_k |x[r, k] * w~[n, k]|, the scale of the rounding error a row can carry."""
    return np.abs(np.asarray(x_rows, dtype=np.float64)) @ np.abs(np.asarray(w_deq)).T


# ----------------------------------------------------------------------------------
# O6: acceptance bound
# ----------------------------------------------------------------------------------
def ulp(v, dtype: str) -> np.ndarray:
    """Spacing of `dtype` values at |v|: 2^(floor(log2|v|) - p + 1), floored at the
    subnormal spacing (so ulp(0) is the smallest subnormal)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    p = _PRECISION[dtype]
    _, e = np.frexp(v)                  # v = m * 2^e, m in [0.5, 1)  =>  floor(log2 v) = e - 1
    spacing = np.ldexp(1.0, (e - 1) - p + 1)
    return np.where(v > 0, np.maximum(spacing, _SUBNORMAL_SPACING[dtype]),
                    _SUBNORMAL_SPACING[dtype])


def bound(x_rows, w_deq, y_ref, dtype: str) -> np.ndarray:
    """|y - y_ref| <= 4e-3 * sum_k |x_k w~_k| + 0.5 ulp_dtype(y_ref).

    The half-ulp term is the "half a bfloat16 step of a float64 reference" of [mlx-4516]
    (Correctness); the relative term covers float32 accumulation and, for a kernel that
    rounds w~ to the storage dtype first, that rounding (2^-9 < 4e-3 / 2).
    """
    return REL_TOL * abs_products(x_rows, w_deq) + 0.5 * ulp(y_ref, dtype)


def check(y, y_ref, tol) -> dict:
    """Compare kernel output y (float64 view of the dtype values) with y_ref elementwise."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    bad = np.argwhere(~(err <= tol))
    return {"ok": bool(bad.shape[0] == 0), "worst_ratio": worst,
            "n_bad": int(bad.shape[0]), "first_bad": bad[:5].tolist()}


def page_metric(y, ref) -> np.ndarray:
    """Per-row max|y - ref| / max|ref| -- the metric printed by the probe of [issue-47331]
    (Root cause).  Context only; the pass criterion is check()."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(y - ref).max(axis=-1) / np.abs(ref).max(axis=-1)


def reference(x_rows, w_packed, scales_bits, biases_bits, k_cols: int, group_size: int,
              bits: int, dtype: str, rows=None) -> dict:
    """Convenience: unpack -> dequantize -> y_ref and the bound, optionally for a subset
    of output features `rows` (sampled checks at full size)."""
    w_packed = np.asarray(w_packed)
    scales_bits = np.asarray(scales_bits)
    biases_bits = np.asarray(biases_bits)
    if rows is not None:
        w_packed, scales_bits, biases_bits = w_packed[rows], scales_bits[rows], biases_bits[rows]
    codes = unpack(w_packed, bits, k_cols)
    w_deq = dequant(codes, scales_bits, biases_bits, group_size, dtype)
    y_ref = matmul_rows(x_rows, w_deq)
    return {"y_ref": y_ref, "tol": bound(x_rows, w_deq, y_ref, dtype), "w_deq": w_deq}


# ----------------------------------------------------------------------------------
# gathered weights (expert-indexed rows)
# ----------------------------------------------------------------------------------
def gather_reference(x_rows, experts, index, k_cols: int, group_size: int, bits: int,
                     dtype: str) -> dict:
    """Expert-indexed decode ([mlx-4516], pull request text: "Gathered QMV"; Correctness:
    batched weights): output row r is x_rows[r] times the dequantized weight of expert
    index[r].  `experts` is a list of (w_packed, scales_bits, biases_bits), one per expert.
    Rows whose index lies outside [0, len(experts)) have y_ref = NaN and tol = 0 (the
    library's documented answer for such rows).  Each row goes through `reference` alone."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    index = np.asarray(index)
    n_out = int(np.asarray(experts[0][1]).shape[0])
    y_ref = np.full((x_rows.shape[0], n_out), np.nan)
    tol = np.zeros((x_rows.shape[0], n_out))
    for r in range(x_rows.shape[0]):
        e = int(index[r])
        if 0 <= e < len(experts):
            w_packed, sbits, bbits = experts[e]
            one = reference(x_rows[r:r + 1], w_packed, sbits, bbits, k_cols, group_size, bits, dtype)
            y_ref[r] = one["y_ref"][0]
            tol[r] = one["tol"][0]
    return {"y_ref": y_ref, "tol": tol}


# ----------------------------------------------------------------------------------
# dequantization to the storage dtype, embedding rows
# ----------------------------------------------------------------------------------
def dequantize_dtype(codes, scales_bits, biases_bits, group_size: int, dtype: str) -> np.ndarray:
    """Dense dtype weight ([issue-47331] "Root cause": the probe dequantizes back to a dense
    tensor).  Reading taken: one float32 multiply-add then one rounding to dtype, i.e.
    RNE_dtype(RNE_f32(s~ * q + b~)).  s~ * q + b~ is exact in float64 (dequant), and
    numpy's float64 -> float32 cast rounds to nearest even, so the float32 step is that
    single rounding.  Returns the dtype bit patterns."""
    exact = dequant(codes, scales_bits, biases_bits, group_size, dtype)
    return to_dtype_bits(exact.astype(np.float32), dtype)


def embedding_reference(w_packed, scales_bits, biases_bits, indices, k_cols: int, group_size: int,
                        bits: int, dtype: str):
    """Rows indices[r] of the dequantized table, as dtype bit patterns; rows whose index is
    outside [0, N) are None (the library writes NaN there)."""
    w_packed = np.asarray(w_packed)
    n_rows = w_packed.shape[0]
    out = []
    for i in np.asarray(indices):
        i = int(i)
        if 0 <= i < n_rows:
            codes = unpack(w_packed[i:i + 1], bits, k_cols)
            out.append(dequantize_dtype(codes, np.asarray(scales_bits)[i:i + 1], np.asarray(biases_bits)[i:i + 1],
                                        group_size, dtype)[0])
        else:
            out.append(None)
    return out


# ----------------------------------------------------------------------------------
# per-row argmax of the logits
# ----------------------------------------------------------------------------------
def argmax_acceptable(y_ref, tol) -> list:
    """Indices a correct fused argmax may return for each row: every column whose exact
    value could be the largest once each value is allowed its tolerance, i.e.
    y_ref[n] + tol[n] >= max_j (y_ref[j] - tol[j]).  (Several answers are correct when
    logits lie within the tolerance of each other.)"""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    floor = (y_ref - tol).max(axis=1, keepdims=True)
    return [set(np.nonzero(row)[0].tolist()) for row in (y_ref + tol >= floor)]


# ----------------------------------------------------------------------------------
# per-row top-k of the logits
# ----------------------------------------------------------------------------------
def topk_rows(y_bits, k: int, dtype: str):
    """The k largest logits of each row, largest first, from logits held as storage-dtype
    bit patterns (what the decode kernel returns).  Order: larger value first; NaN above
    every number (as the fused argmax counts it); +0 above -0; equal values by lower column
    first, so k = 1 gives the argmax contract's first maximal column.
    Returns (index int64 [rows, k], value float64 [rows, k])."""
    vals = from_dtype_bits(np.asarray(y_bits), dtype)
    rows, n = vals.shape
    idx = np.zeros((rows, k), dtype=np.int64)
    out = np.zeros((rows, k), dtype=np.float64)
    for r in range(rows):
        row = vals[r]

        def rank(j):
            v = row[j]
            if np.isnan(v):
                return (0, 0.0, 0, j)
            return (1, -v, 1 if (v == 0 and np.signbit(v)) else 0, j)

        order = sorted(range(n), key=rank)[:k]
        idx[r] = order
        out[r] = row[order]
    return idx, out
