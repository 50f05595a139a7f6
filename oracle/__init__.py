"""CPU oracle (test infrastructure only): see qmm_oracle.py.  The library never imports it."""
from .qmm_oracle import *  # noqa: F401,F403
from .qmm_oracle import (BF16, FP16, REL_TOL, abs_products, bf16_bits_to_f64, bound, check,
                         dequant, f16_bits_to_f64, f32_to_bf16_bits, f32_to_f16_bits,
                         from_dtype_bits, gather_rows, matmul_rows, pack, page_metric,
                         quantize, reference, to_dtype_bits, ulp, unpack)
