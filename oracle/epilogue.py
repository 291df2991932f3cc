"""The MXFP8 epilogue: a fixed-order sum of fp32 split partials followed by MXFP8 quantisation of
the sum, the output form that production runs on the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give (page "wo_a_w8.py"): the module docstring reports that the MXFP8-epilogue
path is bitwise identical to the stock kernel; in `install`, the dropped-weight path and
`small_mx` hand the fp32 split partials of `_partial_w8` ([S, M, G, N]) to the engine's
`quantize_partial`, which sums them and quantises the result in one kernel, where the plain path
sums them with `_wo_a_reduce` (in ascending split order) and rounds to bf16. The quantiser's own
rule and the order of its sum are not printed.

Readings (each listed in the design notes):
  * the partials are added in fp32, one rounding per addition, in a fixed order given with the
    call: ascending split index, s = 0, 1, ..., S - 1 (the order of `_wo_a_reduce`), or the
    pairwise tree over the split index (splits 2i and 2i + 1 are added, an unpaired last split
    is carried up unchanged, and the level repeats until one value is left);
  * the sum is quantised as an MXFP8 tensor along the output columns: blocks of 32 consecutive
    outputs of one row of the [M, G*N] result (N is a multiple of 32, so no block straddles two
    groups), with the rule of oracle.mx (OCP MX v1.0, E4M3 elements: s = floor(log2 amax) - 8,
    RNE, saturation at 448, E8M0 byte s + 127, NaN byte 255 for a non-finite block);
  * outputs: codes uint8 [M, G*N] and scale bytes uint8 [M, G*N/32], both row-major. The pages'
    consumer takes the scales in a swizzled layout of its own; that layout belongs to the
    consuming kernel and is not reproduced.

gemm_mxfp8_ideal applies the epilogue to the one-step fp32 rounding of the exact float64 GEMM:
the result any exact fp32 summation would quantise. A GPU whose fp32 sums differ from it by the
accumulation order can differ from it only where that difference crosses a rounding boundary.
"""
import numpy as np

from . import formats as F
from .mx import MX_BLOCK, quantize_mx_values
from .ops import gemm_exact_f64

ORDER_ASCENDING = 0
ORDER_PAIRWISE = 1


def sum_partials_f32(part, order):
    """fp32 partials [S, ...] -> their fp32 sum in the given fixed order (float32 additions,
    each rounded to nearest even)."""
    part = np.asarray(part, dtype=np.float32)
    S = part.shape[0]
    if S < 1:
        raise ValueError("at least one partial")
    with np.errstate(invalid="ignore", over="ignore"):     # IEEE inf and NaN results are wanted
        return _sum(part, S, order)


def _sum(part, S, order):
    if order == ORDER_ASCENDING:
        acc = part[0].copy()
        for s in range(1, S):
            acc = (acc + part[s]).astype(np.float32)
        return acc
    if order == ORDER_PAIRWISE:
        level = [part[s] for s in range(S)]
        while len(level) > 1:
            nxt = [(level[2 * i] + level[2 * i + 1]).astype(np.float32) for i in range(len(level) // 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        return level[0].copy()
    raise ValueError(f"unknown order {order}")


def quantize_mx_f32(y):
    """fp32 values [M, L] -> (codes uint8 [M, L], scale bytes uint8 [M, L/32])."""
    y = np.asarray(y, dtype=np.float32)
    if y.ndim != 2 or y.shape[1] % MX_BLOCK:
        raise ValueError("expected [M, L] with L a multiple of 32")
    return quantize_mx_values(y.astype(np.float64))


def reduce_quantize_mx(part, order):
    """The epilogue: partials fp32 [S, M, L] -> MXFP8 codes [M, L] and scale bytes [M, L/32]."""
    return quantize_mx_f32(sum_partials_f32(part, order))


def gemm_mxfp8_ideal(x_bits, G, N, K, q, e):
    """MXFP8 of RNE_fp32(Y_exact), Y viewed as [M, G*N]; also returns Y_exact [M, G, N]."""
    Y = gemm_exact_f64(x_bits, G, N, K, q, e)
    M = Y.shape[0]
    codes, scales = quantize_mx_f32(F.f64_to_fp32(Y).reshape(M, G * N))
    return codes, scales, Y
