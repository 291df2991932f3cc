"""Plain CPU oracle of the small-M block-scaled fp8 weight GEMM and its preparation steps.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU
baseline; never by the product path, and it shares no code with the HIP library.

Sources (the pages):
  * "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py": module docstring, kernels
    _wo_a_partial_w8 and _wo_a_mid_kernel, functions make_twin, wo_a_mid, _dequant_kernel.
  * "recipes/docker-images/mia-tp4/adapter/shared_pad_k.py": docstring sections LOSSLESS and
    WHAT THE PATCH DOES, functions _pad_weight and _pad_input.
  * "recipes/docker-images/mia-tp4/docs/tp4-adapters.md": the draft_head_fp8 row (fp32 logits).

Layouts (the same as the library's):
  x  : bf16 bits, [M, ldx]; group g reads columns [g*K, (g+1)*K)
  q  : e4m3 codes, [G, N, K]
  e  : exponent bytes, [G, N/32, K/32], factor 2^(b-127) for the 32x32 block
  y  : [M, G, N] (bf16 bits or fp32)

Arithmetic: every product bf16 x bf16 is exact in float64 (at most 16 significant bits), the
dot products are summed in float64 (a library matmul), and the result is rounded once, from
float64, to bf16 or fp32. The float64 sum differs from the exact sum by at most
K * 2^-53 * sum|x*w|; the tests pin this oracle against an exact rational brute force.
"""
import numpy as np

from . import formats as F

BLOCK = 32


# ---------------------------------------------------------------------------------------------
# a1: fp32 power-of-two block scales -> exponent bytes
# ---------------------------------------------------------------------------------------------
class ScaleError(ValueError):
    """A block-scale tensor that is not made of positive finite powers of two, or has the
    wrong shape (the shared_pad_k.py page, _pad_weight, refuses both)."""


def scales_from_f32(s, N=None, K=None):
    """fp32 scales [N/32, K/32] -> exponent bytes (the fp32 exponent field).

    A scale is accepted when its fraction bits are zero and it is > 0, as _pad_weight checks
    on the shared_pad_k.py page. Readings where the page is silent: +inf (exponent field 255)
    and NaN are refused too; the subnormal 2^-127 has fraction bits and is refused, as on the
    page. Raises ScaleError on any refused element or on a shape mismatch."""
    s = np.asarray(s)
    if s.dtype != np.float32:
        raise ScaleError("scales must be float32")
    if N is not None and K is not None:
        if N % BLOCK or K % BLOCK or s.shape != (N // BLOCK, K // BLOCK):
            raise ScaleError(f"scale shape {s.shape} does not match a {N}x{K} weight in 32x32 blocks")
    bits = s.view(np.uint32)
    frac = bits & 0x7FFFFF
    efield = (bits >> 23) & 0xFF
    sign = bits >> 31
    good = (frac == 0) & (sign == 0) & (efield >= 1) & (efield <= 254)
    if not np.all(good):
        raise ScaleError(f"{int(np.size(good) - np.count_nonzero(good))} scales are not positive finite powers of two")
    return efield.astype(np.uint8)


# ---------------------------------------------------------------------------------------------
# a4: block dequantisation (weight tile rebuilt as bf16)
# ---------------------------------------------------------------------------------------------
def expand_exponents(e, N, K):
    """[G, N/32, K/32] exponent bytes -> [G, N, K] float64 factors 2^(b-127)."""
    f = F.exp_factor(e)
    return np.repeat(np.repeat(f, BLOCK, axis=1), BLOCK, axis=2)[:, :N, :K]


def dequant_values(q, e):
    """Effective weight: bf16(decode(q) * 2^(b-127)), one RNE rounding from the exact product.
    (wo_a_w8.py page: the in-register rebuild in _wo_a_partial_w8 / _wo_a_mid_kernel and the
    standalone _dequant_kernel.) Returns float64 values that bf16 represents exactly."""
    q = np.asarray(q, dtype=np.uint8)
    G, N, K = q.shape
    vals = F.decode_e4m3(q) * expand_exponents(e, N, K)   # exact: power-of-two factor
    return F.round_bf16(vals)


def dequant_bf16(q, e):
    """Same as dequant_values, as bf16 bit patterns [G, N, K] (the DROP path's bf16 copy)."""
    return F.f64_to_bf16_bits(dequant_values(q, e))


# ---------------------------------------------------------------------------------------------
# a5-a7: the GEMM, Y[m, g, n] = sum_k X[m, g*K + k] * W[g, n, k]
# ---------------------------------------------------------------------------------------------
def gemm_exact_f64(x_bits, G, N, K, q, e):
    """float64 Y [M, G, N] before the output rounding. NaN weight codes are refused: the
    configurations exclude them and an exact oracle has nothing to say about them."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape != (G, N, K):
        raise ValueError(f"q shape {q.shape} != {(G, N, K)}")
    if np.isin(q, F.E4M3_NAN_CODES).any():
        raise ValueError("NaN weight code")
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    if x_bits.shape[1] < G * K:
        raise ValueError("ldx < G*K")
    X = F.bf16_bits_to_f64(x_bits[:, : G * K]).reshape(M, G, K)
    W = dequant_values(q, e)
    Y = np.empty((M, G, N), dtype=np.float64)
    # inf weights give inf * 0 = NaN terms on purpose (the IEEE result the kernels must match)
    with np.errstate(invalid="ignore", over="ignore"):
        for g in range(G):
            Y[:, g, :] = X[:, g, :] @ W[g].T
    return Y


def gemm(x_bits, G, N, K, q, e, out="bf16"):
    """The GEMM with its output rounding: bf16 bits (uint16) or fp32, both RNE in one step
    from float64. The split-K and its fixed reduction order of the pages only change fp32
    rounding; the oracle sums in float64, so it has no split."""
    Y = gemm_exact_f64(x_bits, G, N, K, q, e)
    if out == "bf16":
        return F.f64_to_bf16_bits(Y)
    if out == "f32":
        return F.f64_to_fp32(Y)
    raise ValueError(out)


def abs_products_sum(x_bits, G, N, K, q, e):
    """sum_k |X[m,gK+k] * W[g,n,k]| per output, float64 [M, G, N]: the scale of the fp32
    accumulation error any summation order can make."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    X = np.abs(F.bf16_bits_to_f64(x_bits[:, : G * K]).reshape(M, G, K))
    W = np.abs(dequant_values(q, e))
    S = np.empty((M, G, N), dtype=np.float64)
    for g in range(G):
        S[:, g, :] = X[:, g, :] @ W[g].T
    return S


# ---------------------------------------------------------------------------------------------
# a2: the twin encoder
# ---------------------------------------------------------------------------------------------
def block_exponent(amax):
    """Smallest integer e with max(amax, 2^-126) <= 448 * 2^e, clamped to [-127, 127].

    The wo_a_w8.py page (make_twin) writes this as ceil(log2(max(amax, 2^-126) / 448)); here it
    is found by exact comparisons against 448 * 2^e (exact in float64), starting from a float
    estimate and correcting it, so no logarithm rounding can shift it."""
    a = np.maximum(np.asarray(amax, dtype=np.float64), 2.0 ** -126)
    est = np.ceil(np.log2(a / F.E4M3_MAX)).astype(np.int64)
    for _ in range(3):
        too_small = a > np.ldexp(F.E4M3_MAX, est)              # bound not met: raise e
        est = np.where(too_small, est + 1, est)
        slack = a <= np.ldexp(F.E4M3_MAX, est - 1)             # a smaller e also works
        est = np.where(slack, est - 1, est)
    assert np.all(a <= np.ldexp(F.E4M3_MAX, est)) and np.all(a > np.ldexp(F.E4M3_MAX, est - 1))
    return np.clip(est, -127, 127)


class Twin:
    """Result of make_twin: codes q [G,R,D], exponent bytes e [G,R/32,D/32], per-block ok
    flags [G,R/32,D/32] and the verdict `accepted` (all blocks ok)."""

    def __init__(self, q, e, ok):
        self.q, self.e, self.ok = q, e, ok
        self.accepted = bool(ok.all())


def make_twin(w_bits):
    """bf16 weight bits [G, R, D] (R, D multiples of 32) -> Twin.

    Per 32x32 block (wo_a_w8.py page, make_twin): amax of |w|; block exponent e as in
    block_exponent; q = e4m3 RNE of w * 2^-e; rebuilt tile = bf16(decode(q) * 2^e); the block is
    ok when every rebuilt bit pattern equals the input's. The tensor is accepted when every
    block is ok; the page returns None otherwise. The exponent byte is e + 127.

    Readings where the page is silent:
      * a block holding inf or NaN is never ok; its exponent byte is 255 and its codes are
        0x7F (the e4m3 NaN), so a twin built from it can never pass for a real weight;
      * bitwise equality stands for the page's value equality (the encoder keeps the sign of
        zero, so the two agree here);
      * codes of other rejected blocks are the RNE codes all the same.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    G, R, D = w_bits.shape
    if R % BLOCK or D % BLOCK:
        raise ValueError("R and D must be multiples of 32")
    rb, cb = R // BLOCK, D // BLOCK
    vals = F.bf16_bits_to_f64(w_bits).reshape(G, rb, BLOCK, cb, BLOCK)
    finite = np.isfinite(vals).all(axis=(2, 4))                       # [G, rb, cb]
    amax = np.where(np.isfinite(vals), np.abs(vals), 0.0).max(axis=(2, 4))
    e = block_exponent(amax)                                           # [G, rb, cb]
    e5 = e[:, :, None, :, None]
    scaled = np.ldexp(np.where(np.isfinite(vals), vals, 0.0), -e5)    # exact
    q = F.encode_e4m3(scaled)
    back = F.f64_to_bf16_bits(np.ldexp(F.decode_e4m3(q), e5))
    same = (back == w_bits.reshape(G, rb, BLOCK, cb, BLOCK)).all(axis=(2, 4))
    ok = same & finite
    eb = (e + 127).astype(np.uint8)
    eb = np.where(finite, eb, np.uint8(255)).astype(np.uint8)
    q = np.where(finite[:, :, None, :, None], q, np.uint8(0x7F)).astype(np.uint8)
    return Twin(q.reshape(G, R, D), eb, ok.astype(np.uint8))


# ---------------------------------------------------------------------------------------------
# a3: K padding
# ---------------------------------------------------------------------------------------------
PAD_EXPONENT = 127   # the factor 1.0: the shared_pad_k.py page pads the fp32 scales with ones


def pad_k_weight(q, e, K_pad):
    """q [G,N,K] -> [G,N,K_pad] with zero codes; e [G,N/32,K/32] -> [G,N/32,K_pad/32] with the
    unit exponent 127 (shared_pad_k.py page, _pad_weight)."""
    q = np.asarray(q, dtype=np.uint8)
    e = np.asarray(e, dtype=np.uint8)
    G, N, K = q.shape
    if K_pad < K or K_pad % BLOCK or K % BLOCK:
        raise ValueError("K_pad must be a multiple of 32 and >= K")
    qp = np.zeros((G, N, K_pad), dtype=np.uint8)
    qp[:, :, :K] = q
    ep = np.full((G, N // BLOCK, K_pad // BLOCK), PAD_EXPONENT, dtype=np.uint8)
    ep[:, :, : K // BLOCK] = e
    return qp, ep


def pad_k_input(x_bits, G, K, K_pad):
    """x [M, >=G*K] -> [M, G*K_pad] with a zero tail per group (shared_pad_k.py page,
    _pad_input; the tail is zero)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    out = np.zeros((M, G, K_pad), dtype=np.uint16)
    out[:, :, :K] = x_bits[:, : G * K].reshape(M, G, K)
    return out.reshape(M, G * K_pad)
