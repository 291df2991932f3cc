"""Pins of the oracle GEMM, dequantisation, scale ingestion and K padding (CPU only).

The GEMM is pinned against an exact rational brute force written independently here (its own
e4m3 decode from the bit fields and its own RNE), against one-hot inputs whose products select
single weights, and against integer inputs whose sums are exact in any order."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- independent rational reference ---------------------------------------------------------
def _e4m3_fraction(code):
    s, ef, m = code >> 7, (code >> 3) & 15, code & 7
    assert not (ef == 15 and m == 7)
    mag = Fraction(m, 8) * Fraction(2) ** -6 if ef == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (ef - 7)
    return -mag if s else mag


def _bf16_fraction(bits):
    s, ef, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    assert ef != 0xFF
    mag = Fraction(m, 128) * Fraction(2) ** -126 if ef == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (ef - 127)
    return -mag if s else mag


def _rne_bf16_bits(v):
    """Exact RNE of a Fraction to bf16 bits (zero -> +0; overflow -> infinity)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    qe = max(e, -126) - 7
    n = a / Fraction(2) ** qe
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    if fl == 0:
        return sign
    if qe == -133 and fl < 128:                       # subnormal
        return sign | fl
    if fl == 256:
        fl, qe = 128, qe + 1
    ef = qe + 7 + 127
    if ef >= 255:
        return sign | 0x7F80                         # overflow rounds to infinity
    assert ef >= 1
    return sign | (ef << 7) | (fl - 128)


def _brute_gemm_bits(x, G, N, K, q, e):
    M = x.shape[0]
    out = np.zeros((M, G, N), dtype=np.uint16)
    for m in range(M):
        for g in range(G):
            xs = [_bf16_fraction(int(x[m, g * K + k])) for k in range(K)]
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    if xs[k] == 0:
                        continue
                    w = _e4m3_fraction(int(q[g, n, k])) * Fraction(2) ** (int(e[g, n // 32, k // 32]) - 127)
                    w = _bf16_fraction(_rne_bf16_bits(w))
                    acc += xs[k] * w
                out[m, g, n] = _rne_bf16_bits(acc)
    return out


@pytest.mark.parametrize("seed,M,G,N,K", [(1, 3, 2, 64, 96), (2, 2, 1, 32, 128), (3, 1, 2, 32, 64)])
def test_gemm_equals_exact_rational_brute_force(seed, M, G, N, K):
    r = S.rng(seed)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    # exponents span the extremes: 0 (factor 2^-127, bf16 subnormal results), 254, and typical
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 100, 140)
    e.flat[0] = 0
    e.flat[-1] = 10
    q[0, :32, 32:64] = 0                    # an all-zero block
    y = oracle.gemm(x, G, N, K, q, e)
    want = _brute_gemm_bits(x, G, N, K, q, e)
    nz = want != 0                           # the sign of an exactly-zero sum is not pinned
    assert np.array_equal(y[nz], want[nz])
    assert np.all((y[~nz] & 0x7FFF) == 0)


def test_dequant_equals_rational_brute_force_all_codes_all_exponents():
    codes = np.array([c if c not in (0x7F, 0xFF) else 0 for c in range(256)], dtype=np.uint8)
    q = np.broadcast_to(codes, (1, 32, 256)).copy()
    for b in list(range(0, 16)) + [100, 127, 200, 246, 250, 254]:
        got = oracle.dequant_bf16(q, np.full((1, 1, 8), b, dtype=np.uint8))[0, 0]
        for c in range(256):
            if c in (0x7F, 0xFF):
                continue
            v = _e4m3_fraction(c) * Fraction(2) ** (b - 127)
            want = _rne_bf16_bits(v)
            if c & 0x80 and want == 0:
                want = 0x8000                        # a negative value rounding to zero keeps its sign
            assert int(got[c]) == want, (hex(c), b)


def test_one_hot_rows_select_single_weights():
    # X row m is one-hot at column g*K + k_m: Y[m, g, :] must be the dequantised weight column
    # k_m of group g exactly (this fails for a transposed operand or a wrong group offset)
    G, N, K, M = 2, 64, 96, 4
    r = S.rng(21)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 110, 130)
    W = oracle.dequant_bf16(q, e)
    ks = [0, 17, 63, 95]
    for g in range(G):
        x = np.zeros((M, G * K), dtype=np.uint16)
        for m, k in enumerate(ks):
            x[m, g * K + k] = 0x3F80                 # bf16 1.0
        y = oracle.gemm(x, G, N, K, q, e)
        for m, k in enumerate(ks):
            want = W[g, :, k]
            zero = (want & 0x7FFF) == 0              # the sign of a zero sum is not pinned
            assert np.array_equal(y[m, g][~zero], want[~zero])
            assert np.all((y[m, g][zero] & 0x7FFF) == 0)
            other = 1 - g
            assert np.all((y[m, other] & 0x7FFF) == 0)


def test_integer_exact_regime_matches_integer_matmul():
    G, N, K, M = 2, 64, 256, 5
    r = S.rng(33)
    x = S.small_int_bf16(r, (M, G * K), -4, 4)
    # codes whose values are integers 1..16 and their negatives, exponent byte 127
    int_codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)
                          and oracle.decode_e4m3([c])[0] == int(oracle.decode_e4m3([c])[0])
                          and abs(oracle.decode_e4m3([c])[0]) <= 16], dtype=np.uint8)
    q = int_codes[r.integers(0, int_codes.size, (G, N, K))]
    e = np.full((G, N // 32, K // 32), 127, dtype=np.uint8)
    xi = oracle.bf16_bits_to_f64(x).astype(np.int64).reshape(M, G, K)
    wi = oracle.decode_e4m3(q).astype(np.int64)
    yi = np.stack([xi[:, g] @ wi[g].T for g in range(G)], axis=1)
    y = oracle.gemm(x, G, N, K, q, e, out="f32")
    assert np.array_equal(y.astype(np.int64), yi)


def test_fp32_output_is_one_rounding_of_the_exact_sum():
    G, N, K, M = 1, 32, 64, 2
    r = S.rng(44)
    x = S.bf16_normal(r, (M, K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, 1, 2), 120, 126)
    y = oracle.gemm(x, G, N, K, q, e, out="f32")
    for m in range(M):
        for n in range(N):
            acc = sum(_bf16_fraction(int(x[m, k])) * _bf16_fraction(_rne_bf16_bits(
                _e4m3_fraction(int(q[0, n, k])) * Fraction(2) ** (int(e[0, 0, k // 32]) - 127)))
                for k in range(K))
            # fp32 RNE of the exact sum, via exact comparison with both neighbours
            got = Fraction(float(y[m, 0, n]))
            lo = Fraction(float(np.nextafter(y[m, 0, n], -np.inf)))
            hi = Fraction(float(np.nextafter(y[m, 0, n], np.inf)))
            assert abs(got - acc) <= abs(lo - acc) and abs(got - acc) <= abs(hi - acc)


def test_nan_codes_refused():
    q = np.zeros((1, 32, 32), dtype=np.uint8)
    q[0, 3, 4] = 0x7F
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((1, 32), np.uint16), 1, 32, 32, q, np.full((1, 1, 1), 127, np.uint8))


# ---- a1: scale ingestion ----------------------------------------------------------------------
def test_scales_golden():
    with open(os.path.join(GOLDEN, "scales.txt")) as f:
        rows = [ln.split("#", 1)[0].split() for ln in f if ln.split("#", 1)[0].strip()]
    for hexbits, verdict, byte in rows:
        s = np.array([[int(hexbits, 16)]], dtype=np.uint32).view(np.float32)
        if verdict == "ok":
            assert int(oracle.scales_from_f32(s)[0, 0]) == int(byte), hexbits
        else:
            with pytest.raises(oracle.ScaleError):
                oracle.scales_from_f32(s)


def test_scales_shape_and_dtype_checks():
    s = np.ones((160, 18), np.float32)
    assert oracle.scales_from_f32(s, 5120, 576).shape == (160, 18)
    with pytest.raises(oracle.ScaleError):
        oracle.scales_from_f32(s, 5120, 640)
    with pytest.raises(oracle.ScaleError):
        oracle.scales_from_f32(s.astype(np.float64), 5120, 576)


def test_scales_give_the_same_gemm_as_fp32_factors():
    # Y with exponent bytes from fp32 scales equals Y computed with the fp32 factors directly
    d = S.shared_down(1000, M=2, N=64, K=96)
    e = oracle.scales_from_f32(d["scales"], 64, 96)[None]
    y = oracle.gemm_exact_f64(d["x"], 1, 64, 96, d["q"], e)
    w = oracle.round_bf16(oracle.decode_e4m3(d["q"][0]) *
                          np.repeat(np.repeat(d["scales"].astype(np.float64), 32, 0), 32, 1))
    xf = oracle.bf16_bits_to_f64(d["x"])
    assert np.array_equal(y[:, 0, :], xf @ w.T)


# ---- a3: K padding ----------------------------------------------------------------------------
def test_pad_k_is_bitwise_invariant():
    # shared-expert shape, narrowed in N: K = 576 against K padded to 640 (zero codes, unit
    # exponent, zero input tail) must give identical bits (shared_pad_k.py page, LOSSLESS)
    d = S.shared_down(1001, M=6, N=256, K=576)
    e = oracle.scales_from_f32(d["scales"], 256, 576)[None]
    y576 = oracle.gemm(d["x"], 1, 256, 576, d["q"], e)
    qp, ep = oracle.pad_k_weight(d["q"], e, 640)
    xp = oracle.pad_k_input(d["x"], 1, 576, 640)
    y640 = oracle.gemm(xp, 1, 256, 640, qp, ep)
    assert np.array_equal(y576, y640)
    assert np.all(qp[:, :, 576:] == 0) and np.all(ep[:, :, 18:] == 127)
    assert np.all(xp[:, 576:] == 0) and np.array_equal(xp[:, :576], d["x"])
    # the pad exponent does not matter: zero codes times any factor are zero
    for b in (0, 200):
        ep2 = ep.copy()
        ep2[:, :, 18:] = b
        assert np.array_equal(oracle.gemm(xp, 1, 256, 640, qp, ep2), y576)


def test_pad_k_input_groups():
    r = S.rng(5)
    x = S.bf16_normal(r, (3, 2 * 64 + 8))         # ldx larger than G*K
    xp = oracle.pad_k_input(x, 2, 64, 96)
    assert xp.shape == (3, 192)
    assert np.array_equal(xp[:, :64], x[:, :64]) and np.array_equal(xp[:, 96:160], x[:, 64:128])
    assert np.all(xp[:, 64:96] == 0) and np.all(xp[:, 160:] == 0)
