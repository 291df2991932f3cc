"""Number formats used by the block-scaled fp8 weight path, written out from their definitions.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path never does.

Every value here is computed in float64 and rounded ONCE to the target format with
round-half-to-even (RNE). Nothing is taken from a GPU or from the library under test.

Formats:
  * e4m3 ("float8_e4m3fn", the weight code of the wo_a_w8.py page, function make_twin):
    1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent field 0 holds the
    subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN; there is no infinity;
    the largest finite magnitude is 1.75 * 2^8 = 448.
  * bf16: the top half of an IEEE binary32 (8 exponent bits, 7 fraction bits).
  * the block exponent byte b stands for the factor 2^(b - 127) (the exponent tensor of the
    wo_a_w8.py page, kernel _wo_a_partial_w8 and make_twin: the byte is e + 127).
"""
import math

import numpy as np

E4M3_MAX = 448.0
BF16_EMIN = -126          # exponent of the smallest normal bf16 / fp32
BF16_EMAX = 127
BF16_FRAC = 7
FP32_FRAC = 23
E4M3_EMIN = -6            # exponent field 1 with bias 7
E4M3_EMAX = 8
E4M3_FRAC = 3


def _e4m3_value(code):
    """Value of one e4m3fn code, straight from the bit fields."""
    sign = code >> 7
    efield = (code >> 3) & 0xF
    frac = code & 0x7
    if efield == 0xF and frac == 0x7:
        return math.nan
    if efield == 0:
        mag = frac * 2.0 ** -9                       # subnormal: 0.fff * 2^(1-7)
    else:
        mag = (1.0 + frac / 8.0) * 2.0 ** (efield - 7)
    return -mag if sign else mag


# 256-entry decode table, built from the bit-field definition above.
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_NAN_CODES = (0x7F, 0xFF)


def decode_e4m3(codes):
    """e4m3 codes (uint8 array) -> exact float64 values (NaN codes give NaN)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def exp_factor(b):
    """Exponent byte b in [0, 254] -> 2^(b-127), exact in float64. Byte 255 is refused:
    the pages never produce it (make_twin clamps e to [-127, 127])."""
    b = np.asarray(b)
    if b.size and (b.min() < 0 or b.max() > 254):
        raise ValueError("exponent byte outside [0, 254]")
    return np.ldexp(1.0, b.astype(np.int64) - 127)


def round_to_binary(x, frac_bits, emin, emax, overflow="inf"):
    """Round float64 values to a binary floating-point format, round-half-to-even, once.

    The format has `frac_bits` stored fraction bits, smallest normal exponent `emin`, largest
    exponent `emax`, and gradual underflow (subnormals with quantum 2^(emin - frac_bits)).
    Returns float64 values that the format represents exactly. Results beyond the largest
    finite value become +-inf (overflow="inf") or raise (overflow="raise"). Signs of zeros
    are kept; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    finite = np.isfinite(mag)
    safe = np.where(finite, mag, 0.0)
    _, e2 = np.frexp(safe)                     # safe = f * 2^e2 with f in [0.5, 1)
    lead = e2.astype(np.int64) - 1             # exponent of the leading bit
    quantum = np.maximum(lead, emin) - frac_bits
    # scaling by a power of two is exact in float64; rint rounds half to even
    n = np.rint(np.ldexp(safe, -quantum))
    r = np.ldexp(n, quantum)
    largest = (2.0 - 2.0 ** -frac_bits) * 2.0 ** emax
    over = r > largest
    if np.any(over & finite):
        if overflow == "raise":
            raise OverflowError("value beyond the format's largest finite magnitude")
        r = np.where(over, np.inf, r)
    r = np.where(finite, r, mag)
    return np.copysign(r, x)


def round_bf16(x):
    """float64 -> bf16-representable float64 (RNE, one rounding)."""
    return round_to_binary(x, BF16_FRAC, BF16_EMIN, BF16_EMAX)


def round_fp32(x):
    """float64 -> fp32-representable float64 (RNE, one rounding)."""
    return round_to_binary(x, FP32_FRAC, BF16_EMIN, BF16_EMAX)


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> bf16 bit patterns, RNE in one step from float64 (never through fp32).
    NaN maps to the quiet pattern 0x7FC0 (sign kept)."""
    r = round_bf16(x)
    # r is a bf16 value, hence exactly an fp32 value: the cast below is exact
    with np.errstate(invalid="ignore", over="ignore"):
        u = np.asarray(r, dtype=np.float32).view(np.uint32)
    hi = (u >> 16).astype(np.uint16)
    nan = np.isnan(r)
    if np.any(nan):
        hi = np.where(nan, (hi & 0x8000) | 0x7FC0, hi).astype(np.uint16)
    return hi


def f64_to_fp32(x):
    """float64 -> float32 array, RNE in one step (exact cast of the rounded value)."""
    return np.asarray(round_fp32(x), dtype=np.float32)


# Codes 0x00..0x7E hold the non-negative finite values in increasing order, so the code of a
# representable magnitude is its position in that run; the sign bit adds 0x80.
_E4M3_POS = E4M3_TABLE[:0x7F]


def encode_e4m3(x):
    """float64 values with |x| <= 448 after rounding -> e4m3 codes, RNE (ties to the even code).
    Values below 2^-10 in magnitude round to a signed zero. Raises on NaN or overflow: the
    encoder of make_twin never produces either, by construction of its block exponent."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no e4m3 encoding here")
    r = round_to_binary(x, E4M3_FRAC, E4M3_EMIN, E4M3_EMAX, overflow="raise")
    mag = np.abs(r)
    if np.any(mag > E4M3_MAX):
        raise OverflowError("e4m3 overflow")
    pos = np.searchsorted(_E4M3_POS, mag)
    if not np.array_equal(_E4M3_POS[pos], mag):
        raise AssertionError("rounded value is not an e4m3 value")
    sign = np.signbit(r).astype(np.uint8) << 7
    return (pos.astype(np.uint8) | sign).astype(np.uint8)
