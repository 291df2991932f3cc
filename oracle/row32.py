"""Per-(row, 32-column) scale variant of the twin and of the GEMM: a "next" step after the 32x32
block path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row draft_main_proj: each rank
keeps its 1280 output columns of the draft's main projection as e4m3 values with one power-of-two
scale per row and 32 consecutive columns, checked to reproduce the weight exactly, and a GEMV
computes them from the bf16 activation for up to 16 rows.

Reading: the page gives the granularity and the exactness check, not the encoder. The per-block
rule here is the 32x32 twin's (oracle.ops.make_twin, page "wo_a_w8.py", make_twin) applied to
1x32 blocks: least exponent e with max(amax, 2^-126) <= 448 * 2^e, clamped to [-127, 127];
e4m3 codes by one RNE rounding of w * 2^-e; the block is exact when bf16(e4m3(q) * 2^e) equals w
bit for bit; exponent byte e + 127; a block holding inf or NaN is never exact and gets byte 255
and codes 0x7F.

Layouts: weight bits [G, N, K]; codes q [G, N, K]; exponent bytes e [G, N, K/32] (one per row and
32 columns). The GEMM is the one of oracle.ops.gemm with these weights: float64 products and sums,
one rounding to bf16 or fp32.
"""
import numpy as np

from . import formats as F
from .ops import BLOCK, Twin, block_exponent


def expand_row_exponents(e, K):
    """[G, N, K/32] exponent bytes -> [G, N, K] float64 factors 2^(b-127)."""
    return np.repeat(F.exp_factor(e), BLOCK, axis=2)[:, :, :K]


def dequant_values_row32(q, e):
    """bf16(decode(q) * 2^(b-127)) with one exponent per row and 32 columns, rounded once
    (float64 values that bf16 represents exactly)."""
    q = np.asarray(q, dtype=np.uint8)
    G, N, K = q.shape
    e = np.asarray(e, dtype=np.uint8)
    if e.shape != (G, N, K // BLOCK):
        raise ValueError(f"exponent shape {e.shape} != {(G, N, K // BLOCK)}")
    return F.round_bf16(F.decode_e4m3(q) * expand_row_exponents(e, K))


def dequant_bf16_row32(q, e):
    return F.f64_to_bf16_bits(dequant_values_row32(q, e))


def gemm_exact_f64_row32(x_bits, G, N, K, q, e):
    """float64 Y [M, G, N] = sum_k X[m, g*K + k] * W[g, n, k] before the output rounding
    (NaN weight codes refused)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape != (G, N, K):
        raise ValueError(f"q shape {q.shape} != {(G, N, K)}")
    if np.isin(q, F.E4M3_NAN_CODES).any():
        raise ValueError("NaN weight code")
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    X = F.bf16_bits_to_f64(x_bits[:, : G * K]).reshape(M, G, K)
    W = dequant_values_row32(q, e)
    Y = np.empty((M, G, N), dtype=np.float64)
    for g in range(G):
        Y[:, g, :] = X[:, g, :] @ W[g].T
    return Y


def gemm_row32(x_bits, G, N, K, q, e, out="bf16"):
    Y = gemm_exact_f64_row32(x_bits, G, N, K, q, e)
    if out == "bf16":
        return F.f64_to_bf16_bits(Y)
    if out == "f32":
        return F.f64_to_fp32(Y)
    raise ValueError(out)


def abs_products_sum_row32(x_bits, G, N, K, q, e):
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    X = np.abs(F.bf16_bits_to_f64(x_bits[:, : G * K]).reshape(M, G, K))
    W = np.abs(dequant_values_row32(q, e))
    S = np.empty((M, G, N), dtype=np.float64)
    for g in range(G):
        S[:, g, :] = X[:, g, :] @ W[g].T
    return S


def make_twin_row32(w_bits):
    """bf16 weight bits [G, N, K] (K a multiple of 32) -> Twin with q [G, N, K], e and ok
    [G, N, K/32] (one block per row and 32 columns), accepted when every block is exact."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    G, N, K = w_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    cb = K // BLOCK
    vals = F.bf16_bits_to_f64(w_bits).reshape(G, N, cb, BLOCK)
    finite = np.isfinite(vals).all(axis=3)                             # [G, N, cb]
    amax = np.where(np.isfinite(vals), np.abs(vals), 0.0).max(axis=3)
    e = block_exponent(amax)                                           # [G, N, cb]
    scaled = np.ldexp(np.where(np.isfinite(vals), vals, 0.0), -e[..., None])   # exact
    q = F.encode_e4m3(scaled)
    back = F.f64_to_bf16_bits(np.ldexp(F.decode_e4m3(q), e[..., None]))
    same = (back == w_bits.reshape(G, N, cb, BLOCK)).all(axis=3)
    ok = same & finite
    eb = np.where(finite, (e + 127).astype(np.uint8), np.uint8(255)).astype(np.uint8)
    q = np.where(finite[..., None], q, np.uint8(0x7F)).astype(np.uint8)
    return Twin(q.reshape(G, N, K), eb, ok.astype(np.uint8))
