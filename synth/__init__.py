"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and lays them out; it holds none of the quantization or
matmul arithmetic (that lives in the library and, independently, in the oracle).  All
draws use torch's CPU generator with an explicit seed, so they are identical on every
machine; callers move the tensors to the device themselves.

Workloads (shapes of the pages' cases, values synthetic):
  probe    W [1024, 2048] ~ N(0,1), seed 0 (the issue-47331 kernel probe's construction),
           4-bit, group 64, bf16; x ~ N(0,1) in [2,K], [2,1,K], [2,4,K].
  decode   batched decode projections (K, N) in {(1024,2048), (1024,1024), (1024,3072),
           (3072,1024)}, 4 and 8 bits, group 64, bf16; W ~ N(0, 0.02); x [B,1,K], B <= 32.
  lm_head  x [32,1,1024] ~ N(0,1), W [151936, 1024] ~ N(0, 0.02), 4-bit, group 64, bf16.
  odd_n    K = 4096, N in {1,4,7,13,1001}, bits {2,3,5,6}, group {32,64,128}, fp16/bf16,
           x alternating 2048, 1; codes constructed (see odd_n_weight).
  prefill  x [4,512,4096] ~ N(0,1) (and a view narrowed on dim 1 of [4,1024,4096]),
           W [14336, 4096] ~ N(0, 0.02), 4-bit, group 128, bf16.
  experts  a stack of 128 experts of [704, 1408], 8-bit, group 32, bf16 (the expert tensor
           shapes of the Bits=8 report, section 4.3); 128 decode rows, row r routed to
           expert perm[r] of a seeded permutation, so every expert is read once.
  embed    the lm_head table [151936, 1024] 4-bit group 64 read as a tied embedding: 2048
           seeded token indices.
  unaligned the prefill weight at K = 4128 (4096 + 32), group 32: x [4,512,4128].
"""
from __future__ import annotations

import numpy as np
import torch

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def normal_weight(n: int, k: int, std: float, seed: int) -> torch.Tensor:
    """float32 [n, k] ~ N(0, std^2)."""
    w = torch.randn(n, k, generator=_gen(seed), dtype=torch.float32)
    return w * std if std != 1.0 else w


def probe_weight() -> torch.Tensor:
    """The issue-47331 probe's weight: seed 0, then randn(N=1024, K=2048)."""
    return torch.randn(1024, 2048, generator=_gen(0), dtype=torch.float32)


def normal_x(shape, dtype: str, seed: int) -> torch.Tensor:
    """Activations ~ N(0,1), drawn in float32 and stored in `dtype`."""
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32).to(TORCH_DTYPE[dtype])


def alternating_x(k: int, dtype: str, big: float = 2048.0, small: float = 1.0) -> torch.Tensor:
    """[1, k] with x[2j] = big and x[2j+1] = small: a running sum kept in half precision
    drops every `small` (big + small rounds back to big)."""
    x = torch.empty(1, k, dtype=torch.float32)
    x[:, 0::2] = big
    x[:, 1::2] = small
    return x.to(TORCH_DTYPE[dtype])


def odd_n_weight(n: int, k: int, bits: int, group_size: int, seed: int,
                 first_row_zero: bool = False) -> dict:
    """Constructed codes with exactly representable scales and biases.

    Every (row, group) gets s = 2^-13 and a code c_g drawn uniformly from [1, 2^bits - 1],
    with bias b = -c_g * s.  Rows alternate between two kinds:
      * "random": codes uniform in [0, 2^bits - 1];
      * "zero":   every code equals c_g, so every dequantized weight s*q + b is exactly 0
                  and the exact product is 0, while s * sum(x*q) and b * sum(x) are large.
    Returns codes (uint8 [n, k]), scale/bias values (float32 [n, G], exact in bf16 and fp16)
    and the boolean row-kind mask `zero_rows`.
    """
    g = _gen(seed)
    qmax = (1 << bits) - 1
    n_groups = k // group_size
    c = torch.randint(1, qmax + 1, (n, n_groups), generator=g, dtype=torch.int64)
    rand_codes = torch.randint(0, qmax + 1, (n, k), generator=g, dtype=torch.int64)
    zero_rows = (torch.arange(n) % 2 == (0 if first_row_zero else 1))
    const_codes = c.repeat_interleave(group_size, dim=1)
    codes = torch.where(zero_rows[:, None], const_codes, rand_codes)
    s = torch.full((n, n_groups), 2.0 ** -13, dtype=torch.float32)
    b = -(c.to(torch.float32) * s)
    return {"codes": codes.to(torch.uint8).numpy(), "scale_values": s.numpy(),
            "bias_values": b.numpy(), "zero_rows": zero_rows.numpy()}


DECODE_SHAPES = [(1024, 2048), (1024, 1024), (1024, 3072), (3072, 1024)]
DECODE_BATCHES = [1, 2, 4, 8, 16, 32]
ODD_N = [1, 4, 7, 13, 1001]
ODD_BITS = [2, 3, 5, 6]
GROUPS = [32, 64, 128]
LM_HEAD = {"n": 151936, "k": 1024, "m": 32, "bits": 4, "group_size": 64, "dtype": "bf16",
           "w_seed": 300, "x_seed": 301, "w_std": 0.02}
PREFILL = {"n": 14336, "k": 4096, "b": 4, "s": 512, "bits": 4, "group_size": 128,
           "dtype": "bf16", "w_seed": 500, "x_seed": 501, "buf_seed": 502, "w_std": 0.02}


EXPERTS = {"e": 128, "n": 704, "k": 1408, "bits": 8, "group_size": 32, "dtype": "bf16",
           "rows": 128, "w_seed": 700, "x_seed": 701, "idx_seed": 702, "w_std": 0.02}
EMBED = {"count": 2048, "idx_seed": 801}
UNALIGNED = {"n": 14336, "k": 4128, "b": 4, "s": 512, "bits": 4, "group_size": 32,
             "dtype": "bf16", "w_seed": 900, "x_seed": 901, "w_std": 0.02}


def random_packed_weight(n: int, row_words: int, groups: int, dtype: str, seed: int, scale_std: float = 1e-3,
                         bias_std: float = 1e-3):
    """A packed weight drawn directly, for shapes too large to quantize on the host: int32
    [n, row_words] words with every bit pattern equally likely (so every code value occurs),
    scales ~ N(0, scale_std^2) and biases ~ N(0, bias_std^2) [n, groups], stored in dtype."""
    g = _gen(seed)
    words = torch.randint(-2 ** 31, 2 ** 31, (n, row_words), generator=g, dtype=torch.int64).to(torch.int32)
    scales = (torch.randn(n, groups, generator=g, dtype=torch.float32) * scale_std).to(TORCH_DTYPE[dtype])
    biases = (torch.randn(n, groups, generator=g, dtype=torch.float32) * bias_std).to(TORCH_DTYPE[dtype])
    return words, scales, biases


def permutation(n: int, seed: int) -> torch.Tensor:
    """int32 seeded permutation of range(n)."""
    return torch.randperm(n, generator=_gen(seed)).to(torch.int32)


def token_indices(count: int, n: int, seed: int) -> torch.Tensor:
    """int32 [count] uniform in [0, n)."""
    return torch.randint(0, n, (count,), generator=_gen(seed), dtype=torch.int64).to(torch.int32)


def rows_sample(n: int, count: int, seed: int) -> np.ndarray:
    """A sorted random subset of output rows that always includes the first and last rows."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def tied_logits(rows: int, n: int, levels: int, dtype: str, seed: int) -> torch.Tensor:
    """[rows, n] integer-valued logits in [-levels, levels] (many exact ties), in dtype."""
    v = torch.randint(-levels, levels + 1, (rows, n), generator=_gen(seed), dtype=torch.int64)
    return v.to(torch.float32).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
