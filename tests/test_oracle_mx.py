"""Pins of the MXFP8 oracle (oracle/mx.py) against what the format definitions and the
mathematics fix: an integer rule for the scale over every bf16 magnitude, exhaustive nearest-code
search with exact rationals, worked blocks, scaling invariance, round trips of representable
blocks, and an exact rational brute force of the contraction (also tied to the pinned bf16 GEMM
oracle when the activations are already MX values)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.mx as MX
import synthetic as S


def _bits(vals):
    """float values exactly representable in bf16 -> bf16 bits."""
    return oracle.f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))


def test_scale_exponent_integer_rule_over_every_bf16_magnitude():
    # every positive finite bf16 pattern: floor(log2(v)) from the bit fields, then - 8, clamped
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    E = (bits.astype(np.int64) >> 7) & 0xFF
    m = bits.astype(np.int64) & 0x7F
    lead = np.where(E > 0, E - 127, np.floor(np.log2(np.maximum(m, 1))).astype(np.int64) - 133)
    want = np.clip(lead - 8, -127, 127)
    assert np.array_equal(MX.mx_scale_exponent(v), want)
    assert MX.mx_scale_exponent(0.0) == -127


def _nearest_code_exact(t):
    """Brute force: the e4m3 code nearest to the rational t (ties to the code with an even last
    bit), saturating beyond 448; signed zero kept."""
    mag = abs(t)
    best = None
    for c in range(0x7F):                        # non-negative finite codes, ascending
        val = Fraction(float(oracle.decode_e4m3(np.uint8(c))))
        d = abs(val - mag)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    # beyond 448 the saturating conversion keeps 448 (a value past the midpoint 464 would round
    # to 480, which e4m3fn does not have)
    c = best[1]
    return (0x80 | c) if t < 0 else c


def test_element_rounding_matches_exhaustive_search():
    r = S.rng(71)
    for trial in range(60):
        x = S.bf16_normal(r, (1, 32))
        if trial % 3 == 1:
            x = _bits(oracle.bf16_bits_to_f64(x) * 2.0 ** int(r.integers(-40, 40)))
        codes, sc = MX.quantize_mx(x)
        s = int(sc[0, 0]) - 127
        v = oracle.bf16_bits_to_f64(x[0])
        for i in range(32):
            t = Fraction(float(v[i])) / Fraction(2) ** s if s >= 0 else Fraction(float(v[i])) * Fraction(2) ** (-s)
            want = _nearest_code_exact(t)
            if v[i] == 0:
                want = 0x80 if np.signbit(v[i]) else 0
            assert codes[0, i] == want, (trial, i, float(t), hex(codes[0, i]), hex(want))


def test_worked_blocks():
    # all ones: floor(log2 1) = 0 -> s = -8 (byte 119); 1 * 2^8 = 256 = code 0x78
    c, s = MX.quantize_mx(_bits([1.0] * 32)[None])
    assert s[0, 0] == 119 and np.all(c == 0x78)
    # max 14 = 1.75 * 2^3: s = -5, 14 * 32 = 448 exactly (0x7E); 0.5 * 32 = 16 = 0x58
    c, s = MX.quantize_mx(_bits([14.0, 0.5] + [0.0] * 30)[None])
    assert s[0, 0] == 122 and c[0, 0] == 0x7E and c[0, 1] == 0x58
    # max 15 = 1.875 * 2^3: 15 * 32 = 480 is past 448, the conversion saturates at 448
    c, s = MX.quantize_mx(_bits([15.0, -15.0] + [1.0] * 30)[None])
    assert s[0, 0] == 122 and c[0, 0] == 0x7E and c[0, 1] == 0xFE
    # 463 and 464 after scaling: 463 rounds to 448, the tie 464 goes to the even code 448
    c, _ = MX.quantize_mx(_bits([1.80859375, 1.8125] + [0.0] * 30)[None])   # x 256 = 463, 464
    assert c[0, 0] == 0x7E and c[0, 1] == 0x7E
    # the smallest bf16 subnormal: floor(log2) = -133, s clamps at -127, 2^-133 * 2^127 = 2^-6
    c, s = MX.quantize_mx(_bits([2.0 ** -133] + [0.0] * 31)[None])
    assert s[0, 0] == 0 and c[0, 0] == 0x08
    # all-zero block (signs kept) and a non-finite block
    c, s = MX.quantize_mx(_bits([0.0, -0.0] * 16)[None])
    assert s[0, 0] == 0 and c[0, 0] == 0x00 and c[0, 1] == 0x80
    c, s = MX.quantize_mx(_bits([np.inf, -1.0] + [1.0] * 30)[None])
    assert s[0, 0] == 255 and c[0, 0] == 0x7F and c[0, 1] == 0xFF


def test_scaling_by_powers_of_two_moves_only_the_scale():
    r = S.rng(72)
    x = S.bf16_normal(r, (8, 256))
    c0, s0 = MX.quantize_mx(x)
    for j in (-20, -1, 1, 13):
        cj, sj = MX.quantize_mx(_bits(oracle.bf16_bits_to_f64(x) * 2.0 ** j))
        assert np.array_equal(cj, c0) and np.array_equal(sj.astype(int), s0.astype(int) + j)


def test_representable_blocks_round_trip():
    # blocks built as code * 2^s with the block maximum in the top binade [256, 448] are exactly
    # representable and must come back unchanged
    r = S.rng(73)
    M, L = 6, 256
    codes = S.e4m3_codes(r, (M, L))
    blocks = codes.reshape(M, L // 32, 32)
    blocks[:, :, 0] = r.integers(0x78, 0x7F, size=(M, L // 32)).astype(np.uint8)   # 256..448
    mag = blocks & 0x7F
    top = mag.max(axis=2)
    assert np.all(top >= 0x78)
    s = r.integers(-30, 20, size=(M, L // 32))
    vals = oracle.decode_e4m3(blocks) * np.ldexp(1.0, s)[:, :, None]
    x = _bits(vals.reshape(M, L))
    assert np.array_equal(oracle.bf16_bits_to_f64(x), vals.reshape(M, L))
    cq, sq = MX.quantize_mx(x)
    assert np.array_equal(sq.astype(int) - 127, s)
    assert np.array_equal(MX.dequant_mx(cq, sq), vals.reshape(M, L))


def test_dequant_error_within_half_an_e4m3_ulp():
    r = S.rng(74)
    x = S.bf16_normal(r, (16, 512))
    cq, sq = MX.quantize_mx(x)
    v = oracle.bf16_bits_to_f64(x)
    d = MX.dequant_mx(cq, sq)
    s = np.repeat(sq.astype(np.int64) - 127, 32, axis=1)
    t = np.abs(v) * np.ldexp(1.0, -s)                    # scaled magnitudes, < 512
    sat = t > 464
    normal = (t >= 2.0 ** -6) & ~sat
    rel = np.abs(d - v)[normal] / np.abs(v)[normal]
    assert rel.max() <= 2.0 ** -4
    assert np.all(np.abs(d[sat]) == np.ldexp(448.0, s[sat]))


def _brute_gemm_mx(xq, xs, G, N, K, q, e):
    """Exact rational Y from the bit fields (own decode of both operands)."""
    def dec(c):
        s = -1 if c & 0x80 else 1
        E, f = (c >> 3) & 15, c & 7
        mag = Fraction(f, 8) * Fraction(1, 64) if E == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (E - 7)
        return s * mag
    def p2(b):
        return Fraction(2) ** (int(b) - 127) if b >= 127 else Fraction(1, 2 ** (127 - int(b)))
    M = xq.shape[0]
    Y = np.empty((M, G, N), dtype=object)
    for m in range(M):
        for g in range(G):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    xv = dec(int(xq[m, g * K + k])) * p2(xs[m, (g * K + k) // 32])
                    wv = dec(int(q[g, n, k])) * p2(e[g, n // 32, k // 32])
                    acc += xv * wv
                Y[m, g, n] = acc
    return Y


@pytest.mark.parametrize("M,G,N,K,seed", [(2, 1, 32, 64, 75), (3, 2, 32, 96, 76)])
def test_gemm_mx_exact_brute_force(M, G, N, K, seed):
    r = S.rng(seed)
    x = S.bf16_normal(r, (M, G * K))
    xq, xs = MX.quantize_mx(x)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 100, 140)
    Y = MX.gemm_mx_exact_f64(xq, xs, G, N, K, q, e)
    B = _brute_gemm_mx(xq, xs, G, N, K, q, e)
    got = MX.gemm_mx(xq, xs, G, N, K, q, e, out="bf16")
    for idx in np.ndindex(M, G, N):
        exact = B[idx]
        assert abs(Fraction(float(Y[idx])) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)
        # the bf16 output is the nearest bf16 of the exact value (checked through float64, whose
        # error here is far below a bf16 half ulp)
        assert got[idx] == oracle.f64_to_bf16_bits(float(exact))


def test_gemm_mx_equals_the_bf16_gemm_on_mx_representable_activations():
    # activations that are exactly MX values: the MX contraction and the pinned bf16 GEMM oracle
    # compute the same exact products, so both round to the same bits
    r = S.rng(77)
    M, G, N, K = 4, 2, 64, 256
    codes = S.e4m3_codes(r, (M, G * K)).reshape(M, G * K // 32, 32)
    codes[:, :, 0] = 0x78
    s = r.integers(-20, 5, size=(M, G * K // 32))
    vals = (oracle.decode_e4m3(codes) * np.ldexp(1.0, s)[:, :, None]).reshape(M, G * K)
    x = _bits(vals)
    xq, xs = MX.quantize_mx(x)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 110, 130)
    assert np.array_equal(MX.gemm_mx(xq, xs, G, N, K, q, e), oracle.gemm(x, G, N, K, q, e))
    assert np.array_equal(MX.gemm_mx(xq, xs, G, N, K, q, e, out="f32"), oracle.gemm(x, G, N, K, q, e, out="f32"))
