"""MXFP8 activations and the fp8 x fp8 block-scaled contraction: the first "next" step after the
bf16 hot path, the numerics of the pages' MXFP8 comparison path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give: on the shared_pad_k.py page the MXFP8 linear quantizes its bf16 input itself
when no input scale is passed (the wrapper in `install` refuses an already-quantized input because
the K padding must come before that quantization), and the LOSSLESS section attributes the
behaviour of the padded tail to the MXFP8 quantizer; the quantizer's rule is not printed there. The
rule used here is the one of the OCP Microscaling (MX) formats specification, v1.0, for MXFP8 with
E4M3 elements:
  * a block is 32 consecutive elements of one row (k = 32, the pages' block width as well);
  * the shared scale is an E8M0 power of two 2^s with s = floor(log2(max |v|)) - emax_elem, where
    emax_elem = 8 is the exponent of the largest normal E4M3 number (448 = 1.75 * 2^8);
  * each element is v / 2^s rounded to E4M3 to nearest, ties to even, and clamped to +-448 when
    the rounding goes past the largest normal value (the specification's saturating conversion).
Readings where the specification leaves a choice (each listed in the design notes):
  * s is clamped to the E8M0 range [-127, 127]; an all-zero block gets s = -127 (byte 0) and
    zero codes (signs of zeros kept);
  * a block holding a NaN or an infinity gets the E8M0 NaN byte 255 and NaN codes 0x7F
    (0xFF for negative entries), mirroring the twin encoder's treatment of non-finite blocks.

Layouts: activations x as bf16 bits [M, L] (L = G*K); codes xq uint8 [M, L]; scale bytes xs uint8
[M, L/32] standing for 2^(b - 127). The weights are the twin's e4m3 codes q [G, N, K] and block
exponent bytes e [G, N/32, K/32] exactly as in ops.py: their 32 x 32 block exponent serves as the
MX scale of every row's 32-element piece.

Arithmetic of the contraction: every product of two E4M3 values times two powers of two is exact
in float64; the dot products are summed in float64 and rounded once (as in ops.gemm).
"""
import numpy as np

from . import formats as F
from .ops import dequant_values

MX_BLOCK = 32
E4M3_EMAX_ELEM = 8          # exponent of 448 = 1.75 * 2^8, the largest normal E4M3 value
SCALE_NAN = 255


def mx_scale_exponent(amax):
    """floor(log2(amax)) - 8, clamped to [-127, 127]; amax == 0 gives -127. amax must be finite
    and non-negative. frexp gives amax = f * 2^t with f in [0.5, 1), so floor(log2(amax)) = t - 1
    exactly (no logarithm is evaluated)."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("amax must be finite and non-negative")
    _, t = np.frexp(a)
    s = t.astype(np.int64) - 1 - E4M3_EMAX_ELEM
    s = np.where(a == 0, -127, s)
    return np.clip(s, -127, 127)


def quantize_mx_values(v):
    """float64 values [M, L] (L a multiple of 32; inf and NaN allowed) -> (codes uint8 [M, L],
    scale bytes uint8 [M, L/32]). The values must be exact copies of the inputs (bf16 or fp32
    values are exact in float64), so that every decision below is taken on the input itself."""
    v = np.asarray(v, dtype=np.float64)
    M, L = v.shape
    if L % MX_BLOCK:
        raise ValueError("L must be a multiple of 32")
    v = v.reshape(M, L // MX_BLOCK, MX_BLOCK)
    finite = np.isfinite(v).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(v), v, 0.0)).max(axis=2), 0.0)
    s = mx_scale_exponent(amax)                                   # [M, L/32]
    scaled = np.ldexp(np.where(np.isfinite(v), v, 0.0), -s[:, :, None])   # exact: power of two
    r = F.round_to_binary(scaled, F.E4M3_FRAC, F.E4M3_EMIN, F.E4M3_EMAX, overflow="inf")
    r = np.clip(r, -F.E4M3_MAX, F.E4M3_MAX)                       # saturating conversion
    codes = F.encode_e4m3(r)
    nan_code = np.where(np.signbit(v), 0xFF, 0x7F).astype(np.uint8)
    codes = np.where(finite[:, :, None], codes, nan_code)
    scales = np.where(finite, s + 127, SCALE_NAN).astype(np.uint8)
    return codes.reshape(M, L).astype(np.uint8), scales


def quantize_mx(x_bits, L=None):
    """bf16 bits [M, >= L] -> (codes uint8 [M, L], scale bytes uint8 [M, L/32])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    L = x_bits.shape[1] if L is None else L
    if L % MX_BLOCK:
        raise ValueError("L must be a multiple of 32")
    return quantize_mx_values(F.bf16_bits_to_f64(x_bits[:, :L]))


def dequant_mx(codes, scales):
    """codes [M, L], scale bytes [M, L/32] -> exact float64 values (NaN where a block's scale is
    255 or a code is NaN)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    M, L = codes.shape
    vals = F.decode_e4m3(codes).reshape(M, L // MX_BLOCK, MX_BLOCK)
    fac = np.where(scales == SCALE_NAN, np.nan,
                   np.ldexp(1.0, scales.astype(np.int64) - 127))
    return (vals * fac[:, :, None]).reshape(M, L)


def gemm_mx_exact_f64(xq, xs, G, N, K, q, e):
    """float64 Y [M, G, N] = sum_k Xmx[m, g*K + k] * W[g, n, k], before the output rounding.
    Refuses NaN codes and NaN scales (the oracle has nothing exact to say about them)."""
    xq = np.asarray(xq, dtype=np.uint8)
    xs = np.asarray(xs, dtype=np.uint8)
    M = xq.shape[0]
    if xq.shape[1] < G * K or xs.shape[1] < G * K // MX_BLOCK:
        raise ValueError("activation codes or scales narrower than G*K")
    if np.isin(xq[:, : G * K], F.E4M3_NAN_CODES).any() or (xs[:, : G * K // MX_BLOCK] == SCALE_NAN).any():
        raise ValueError("NaN activation code or scale")
    X = dequant_mx(xq[:, : G * K], xs[:, : G * K // MX_BLOCK]).reshape(M, G, K)
    W = dequant_values(q, e)
    Y = np.empty((M, G, N), dtype=np.float64)
    for g in range(G):
        Y[:, g, :] = X[:, g, :] @ W[g].T
    return Y


def gemm_mx(xq, xs, G, N, K, q, e, out="bf16"):
    """The fp8 x fp8 GEMM with one RNE rounding from float64 to bf16 bits or fp32."""
    Y = gemm_mx_exact_f64(xq, xs, G, N, K, q, e)
    if out == "bf16":
        return F.f64_to_bf16_bits(Y)
    if out == "f32":
        return F.f64_to_fp32(Y)
    raise ValueError(out)


def abs_products_sum_mx(xq, xs, G, N, K, q, e):
    """sum_k |Xmx * W| per output (the scale of any fp32 summation order's error)."""
    xq = np.asarray(xq, dtype=np.uint8)
    M = xq.shape[0]
    X = np.abs(dequant_mx(xq[:, : G * K], np.asarray(xs)[:, : G * K // MX_BLOCK])).reshape(M, G, K)
    W = np.abs(dequant_values(q, e))
    S = np.empty((M, G, N), dtype=np.float64)
    for g in range(G):
        S[:, g, :] = X[:, g, :] @ W[g].T
    return S
