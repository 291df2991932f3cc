"""Pins of the MXFP8 epilogue oracle (oracle/epilogue.py): the fixed-order fp32 sums against exact
rationals and worked cases where the order decides the result, the fp32 quantiser against an
integer exponent rule over every fp32 binade, an exhaustive nearest-code search with exact
rationals (including fp32 values a bf16 cannot hold, at and next to rounding ties), worked blocks,
and the ideal GEMM epilogue against an exact rational brute force."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.epilogue as EP
import oracle.mx as MX
import synthetic as S

ASC, PW = EP.ORDER_ASCENDING, EP.ORDER_PAIRWISE
f32 = np.float32


def _round_f32(fr):
    """Exact rational -> nearest fp32 (ties to even): Fraction -> double is correctly rounded, and
    double -> fp32 after it is the correct rounding of a sum of two fp32 values (53 >= 2*24 + 2)."""
    return f32(float(fr))


def test_order_decides_worked_cases():
    u = 2.0 ** -24                                  # half an ulp of 1.0 in fp32
    p = np.array([[1.0], [u], [u], [u]], dtype=f32)
    # ascending: every 1 + 2^-24 is a tie that goes back to 1
    assert EP.sum_partials_f32(p, ASC)[0] == f32(1.0)
    # pairwise: (1 + u) + (u + u) = 1 + 2^-23, representable
    assert EP.sum_partials_f32(p, PW)[0] == f32(1.0 + 2.0 ** -23)
    # five partials: the tree is [1, 2^-23, u] -> [1 + 2^-23, u] -> the tie 1 + 2^-23 + 2^-24
    # rounds to the even neighbour 1 + 2^-22
    p5 = np.array([[1.0], [u], [u], [u], [u]], dtype=f32)
    assert EP.sum_partials_f32(p5, ASC)[0] == f32(1.0)
    assert EP.sum_partials_f32(p5, PW)[0] == f32(1.0 + 2.0 ** -22)
    # one partial is returned as it is, in both orders
    one = np.array([[3.5, -0.0]], dtype=f32)
    for o in (ASC, PW):
        r = EP.sum_partials_f32(one, o)
        assert r[0] == f32(3.5) and np.signbit(r[1])
    with pytest.raises(ValueError):
        EP.sum_partials_f32(p, 7)


@pytest.mark.parametrize("S_", [2, 3, 5, 8, 9])
def test_sums_match_exact_rationals_step_by_step(S_):
    r = S.rng(80 + S_)
    part = S.f32_normal(r, (S_, 64)) * np.ldexp(f32(1.0), r.integers(-30, 30, size=(S_, 64))).astype(f32)
    part = part.astype(f32)
    asc = EP.sum_partials_f32(part, ASC)
    pw = EP.sum_partials_f32(part, PW)
    for i in range(part.shape[1]):
        a = part[0, i]
        for s in range(1, S_):
            a = _round_f32(Fraction(float(a)) + Fraction(float(part[s, i])))
        assert asc[i] == a
        lv = [part[s, i] for s in range(S_)]
        while len(lv) > 1:                          # pairs (0,1), (2,3), ...; odd one carried
            nxt = [_round_f32(Fraction(float(lv[j])) + Fraction(float(lv[j + 1]))) for j in range(0, len(lv) - 1, 2)]
            lv = nxt + ([lv[-1]] if len(lv) % 2 else [])
        assert pw[i] == lv[0]


def test_exact_sums_do_not_depend_on_the_order():
    r = S.rng(90)
    part = r.integers(-1000, 1000, size=(7, 5, 96)).astype(f32)
    want = part.astype(np.int64).sum(axis=0)
    for o in (ASC, PW):
        assert np.array_equal(EP.sum_partials_f32(part, o).astype(np.int64), want)


def test_scale_exponent_over_every_fp32_binade():
    r = S.rng(91)
    E = np.repeat(np.arange(0, 255, dtype=np.uint32), 4)
    mant = r.integers(0, 1 << 23, size=E.size).astype(np.uint32)
    bits = (E << 23) | mant
    v = bits.view(f32)
    keep = v > 0
    v, E, mant = v[keep], E[keep], mant[keep]
    # floor(log2 v) read off the fields: E - 127 for a normal, the top set mantissa bit for a subnormal
    lead = np.where(E > 0, E.astype(np.int64) - 127,
                    np.floor(np.log2(np.maximum(mant, 1).astype(np.float64))).astype(np.int64) - 149)
    want = np.clip(lead - 8, -127, 127)
    blocks = np.zeros((v.size, 32), dtype=f32)
    blocks[:, 5] = v
    _, sc = EP.quantize_mx_f32(blocks)
    assert np.array_equal(sc[:, 0].astype(np.int64) - 127, want)


def _nearest_code_exact(t):
    """Brute force: the e4m3 code nearest to the rational t (ties to the even code), saturating
    at 448; the sign of t kept."""
    mag = abs(t)
    best = None
    for c in range(0x7F):
        val = Fraction(float(oracle.decode_e4m3(np.uint8(c))))
        d = abs(val - mag)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return (0x80 | best[1]) if t < 0 else best[1]


def _check_block_exhaustively(vals, codes, scale):
    s = int(scale) - 127
    for i, v in enumerate(vals):
        t = Fraction(float(v)) * (Fraction(2) ** -s if s <= 0 else Fraction(1, 2 ** s))
        want = _nearest_code_exact(t)
        if v == 0:
            want = 0x80 if np.signbit(v) else 0
        assert codes[i] == want, (i, float(v), float(t), hex(codes[i]), hex(want))


def test_fp32_rounding_matches_exhaustive_search():
    r = S.rng(92)
    for trial in range(40):
        v = S.f32_normal(r, (32,)) * f32(2.0 ** int(r.integers(-60, 60)))
        v = v.astype(f32)
        codes, sc = EP.quantize_mx_f32(v[None])
        _check_block_exhaustively(v, codes[0], sc[0, 0])


def test_fp32_values_at_and_next_to_ties():
    # block maximum 1.0: s = -8, scaled value = v * 256. 1.0625 lies halfway between the e4m3
    # values 1.0 (0x38) and 1.125 (0x39): the tie goes to the even code 0x38; one fp32 ulp more
    # (a value no bf16 holds) goes to 0x39, one less to 0x38
    half = f32(1.0625 / 256)
    vals = np.zeros(32, dtype=f32)
    vals[0] = 1.0
    vals[1] = half
    vals[2] = np.nextafter(half, f32(1), dtype=f32)
    vals[3] = np.nextafter(half, f32(0), dtype=f32)
    vals[4] = -vals[2]
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): the tie goes to 0x3A
    vals[5] = f32(1.1875 / 256)
    # 2^-10 after scaling is the tie between 0 and the smallest subnormal 2^-9: to zero; just
    # above it to 0x01
    vals[6] = f32(2.0 ** -18)
    vals[7] = np.nextafter(f32(2.0 ** -18), f32(1), dtype=f32)
    codes, sc = EP.quantize_mx_f32(vals[None])
    assert sc[0, 0] == 119
    assert list(codes[0, :8]) == [0x78, 0x38, 0x39, 0x38, 0xB9, 0x3A, 0x00, 0x01]
    _check_block_exhaustively(vals, codes[0], sc[0, 0])


def test_fp32_worked_blocks():
    # saturation: max 1.9 * 2^4 -> s = -4, 30.4 * 16 = 486.4 > 448 -> 448
    v = np.zeros((1, 32), dtype=f32)
    v[0, 0], v[0, 1] = 30.4, -30.4
    c, s = EP.quantize_mx_f32(v)
    assert s[0, 0] == 123 and c[0, 0] == 0x7E and c[0, 1] == 0xFE
    # fp32 subnormal maximum: floor(log2 2^-140) = -140, s clamps at -127 -> 2^-13, below 2^-10: 0
    v = np.zeros((1, 32), dtype=f32)
    v[0, 3] = np.ldexp(f32(1), -140)
    c, s = EP.quantize_mx_f32(v)
    assert s[0, 0] == 0 and np.all(c == 0)
    # 2^-130 * 2^127 = 2^-3 = code 0x20 (exponent field 4, mantissa 0)
    v[0, 3] = np.ldexp(f32(1), -130)
    c, s = EP.quantize_mx_f32(v)
    assert s[0, 0] == 0 and c[0, 3] == 0x20
    # the largest fp32: floor(log2) = 127 -> s = 119, scaled 1.99.. * 2^8 saturates at 448
    v[0, 3] = np.finfo(f32).max
    c, s = EP.quantize_mx_f32(v)
    assert s[0, 0] == 246 and c[0, 3] == 0x7E
    # non-finite blocks: NaN scale byte and NaN codes with the entries' signs
    v = np.ones((2, 32), dtype=f32)
    v[0, 2] = np.nan
    v[1, 4] = -np.inf
    v[1, 5] = -1.0
    c, s = EP.quantize_mx_f32(v)
    assert list(s[:, 0]) == [255, 255] and c[0, 0] == 0x7F and c[1, 4] == 0xFF and c[1, 5] == 0xFF


def test_fp32_quantizer_equals_the_bf16_one_on_bf16_values():
    r = S.rng(93)
    x = S.bf16_normal(r, (8, 512), scale=3.0)
    v = oracle.bf16_bits_to_f64(x).astype(f32)
    a = EP.quantize_mx_f32(v)
    b = MX.quantize_mx(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_reduce_quantize_is_the_sum_then_the_quantiser():
    r = S.rng(94)
    part = S.f32_normal(r, (4, 3, 128))
    for o in (ASC, PW):
        c, s = EP.reduce_quantize_mx(part, o)
        c2, s2 = EP.quantize_mx_f32(EP.sum_partials_f32(part, o))
        assert np.array_equal(c, c2) and np.array_equal(s, s2)


def _brute_y(x, G, N, K, q, e):
    def dec(c):
        sg = -1 if c & 0x80 else 1
        E, f = (c >> 3) & 15, c & 7
        mag = Fraction(f, 8) * Fraction(1, 64) if E == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (E - 7)
        return sg * mag
    xv = oracle.bf16_bits_to_f64(x)
    M = x.shape[0]
    Y = np.empty((M, G * N), dtype=object)
    for m in range(M):
        for g in range(G):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    b = int(e[g, n // 32, k // 32])
                    w = dec(int(q[g, n, k])) * (Fraction(2) ** (b - 127) if b >= 127 else Fraction(1, 2 ** (127 - b)))
                    # the bf16 rounding of the dequantised weight is exact at these exponents
                    acc += Fraction(float(xv[m, g * K + k])) * w
                Y[m, g * N + n] = acc
    return Y


def test_ideal_epilogue_against_rational_brute_force():
    r = S.rng(95)
    M, G, N, K = 2, 2, 32, 64
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 118, 126)
    codes, scales, Y = EP.gemm_mxfp8_ideal(x, G, N, K, q, e)
    B = _brute_y(x, G, N, K, q, e)
    for m in range(M):
        yf = np.array([_round_f32(B[m, j]) for j in range(G * N)], dtype=f32)
        for b in range(G * N // 32):
            blk = yf[32 * b: 32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            s = int(np.floor(np.log2(amax))) - 8
            assert scales[m, b] == s + 127
            _check_block_exhaustively(blk, codes[m, 32 * b: 32 * b + 32], scales[m, b])


def test_ideal_epilogue_is_exact_on_integer_sums():
    # small-integer activations and integer-valued weights at unit scale: Y is an exact fp32
    # integer, so the ideal epilogue is the quantiser of the exact result
    r = S.rng(96)
    M, G, N, K = 3, 2, 64, 256
    x = S.small_int_bf16(r, (M, G * K))
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53, 0x54, 0x55, 0x56,
                     0x57, 0x58], dtype=np.uint8)          # 0, 1..8, 9..16 in e4m3
    q = ints[r.integers(0, ints.size, size=(G, N, K))] | (r.integers(0, 2, size=(G, N, K)).astype(np.uint8) << 7)
    e = np.full((G, N // 32, K // 32), 127, dtype=np.uint8)
    codes, scales, Y = EP.gemm_mxfp8_ideal(x, G, N, K, q, e)
    assert np.array_equal(Y, np.round(Y)) and np.abs(Y).max() < 2 ** 24
    c2, s2 = EP.quantize_mx_f32(Y.reshape(M, G * N).astype(f32))
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)


def test_parity_rule_of_the_epilogue_catches_a_wrong_code():
    # the GPU-side checker (tests/parity.py) against planted results: the ideal epilogue and the
    # epilogue of fp32 values within the error budget pass; a code one step off where the value
    # is far from a rounding boundary, or a scale one binade off, fails
    from parity import check_mxfp8, rounding_budget, U
    r = S.rng(97)
    M, G, N, K = 3, 1, 64, 256
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 118, 126)
    codes, scales, Y = EP.gemm_mxfp8_ideal(x, G, N, K, q, e)
    Y = Y.reshape(M, G * N)
    A = oracle.abs_products_sum(x, G, N, K, q, e).reshape(M, G * N)
    st = check_mxfp8(codes, scales, Y, A, K, 1)
    assert st["same"] == st["n"]
    noisy = Y + (r.uniform(-1, 1, Y.shape) * rounding_budget(K, 1) * U * A)
    c2, s2 = EP.quantize_mx_f32(oracle.f64_to_fp32(noisy))
    check_mxfp8(c2, s2, Y, A, K, 1)
    # one code one step up at an element whose scaled value is mid-way between two codes
    s_el = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    t = np.abs(np.ldexp(Y, -s_el))
    dec = oracle.decode_e4m3(codes & 0x7F)
    i = np.argmax((np.abs(t - dec) < 1e-3 * np.maximum(dec, 1e-3)) & (t > 16) & (t < 400))
    m, j = divmod(int(i), G * N)
    bad = codes.copy()
    bad[m, j] += 1
    with pytest.raises(AssertionError):
        check_mxfp8(bad, scales, Y, A, K, 1)
    bad_s = scales.copy()
    bad_s[0, 0] += 1
    with pytest.raises(AssertionError):
        check_mxfp8(codes, bad_s, Y, A, K, 1)
