"""CPU oracle for the block-scaled fp8 small-M GEMM path: float64, slow, written from the pages.

TEST INFRASTRUCTURE ONLY. It may be imported by tests/, by __graft_entry__.smoke() and by the
cpu_baseline leg of bench.py, and by nothing else. It shares no code, tables or constants with
the HIP library under block_scaled_fp8_skinny_amd/, and imports nothing from it.

Modules: formats (e4m3, bf16, fp32 rounding), ops (the bf16 hot path and its preparation), mx
(MXFP8 activations and the fp8 x fp8 contraction, the next step after the hot path), row32 (the
per-(row, 32-column) scale twin and its GEMM, another next step), epilogue (the fixed-order sum of
fp32 split partials and MXFP8 quantisation of the output).

Parity status: every function here is pinned by CPU tests (tests/test_oracle_*.py) to values
fixed by the format definitions, closed forms, invariants and exact rational brute force.
"""
from . import formats
from .formats import (bf16_bits_to_f64, decode_e4m3, encode_e4m3, exp_factor, f64_to_bf16_bits,
                      f64_to_fp32, round_bf16, round_fp32, round_to_binary)
from .ops import (PAD_EXPONENT, ScaleError, Twin, abs_products_sum, block_exponent, dequant_bf16,
                  dequant_values, gemm, gemm_exact_f64, make_twin, pad_k_input, pad_k_weight,
                  scales_from_f32)
from . import row32
from . import epilogue
