"""Pins of the oracle's number formats against the format definitions, library casts and exact
rational arithmetic (CPU only)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e4m3_landmarks_golden():
    for code, val in _read_table("e4m3_landmarks.txt"):
        got = oracle.decode_e4m3([int(code, 16)])[0]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_positive_codes_increase():
    v = oracle.decode_e4m3(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)


def test_exp_factor_closed_form():
    assert oracle.exp_factor(127) == 1.0
    assert oracle.exp_factor(0) == 2.0 ** -127
    assert oracle.exp_factor(254) == 2.0 ** 127
    assert oracle.exp_factor(120) == 1.0 / 128
    with pytest.raises(ValueError):
        oracle.exp_factor(255)


def _torch_bf16_bits(f32):
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_fp32_values():
    r = np.random.default_rng(7)
    parts = [r.standard_normal(200000).astype(np.float32),
             (r.standard_normal(20000) * 1e-39).astype(np.float32),        # fp32 subnormals
             np.clip(r.standard_normal(20000) * 3e38, -3.39e38, 3.39e38).astype(np.float32)]  # near overflow
    # exact ties: low 16 bits 0x8000 with both parities of the kept bit
    u = r.integers(0, 2 ** 31, size=20000, dtype=np.uint64).astype(np.uint32)
    u = (u & 0xFFFF0000) | 0x8000
    parts.append(u.view(np.float32))
    x = np.concatenate(parts)
    x = x[np.isfinite(x)]
    ours = oracle.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(ours, _torch_bf16_bits(x))


def _rne_fraction(v, frac_bits, emin, emax):
    """Exact RNE of a Fraction to a binary format (independent brute force); returns Fraction,
    or +-inf as float."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    qe = max(e, emin) - frac_bits
    n = a / Fraction(2) ** qe
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    res = fl * Fraction(2) ** qe
    if res > (2 - Fraction(2) ** -frac_bits) * Fraction(2) ** emax:
        return s * math.inf
    return s * res


def test_bf16_rounding_one_step_from_f64_vs_rational_brute_force():
    r = np.random.default_rng(11)
    # float64 values with many more bits than fp32 keeps, plus hand-made near-ties: a value just
    # above a bf16 tie must round up even though rounding via fp32 first would tie-break down
    xs = list(r.standard_normal(3000) * np.exp2(r.integers(-140, 120, 3000)))
    one_ulp = 2.0 ** -7
    xs += [1 + one_ulp / 2 + 2.0 ** -40, 1 + one_ulp / 2, 1 + 3 * one_ulp / 2, -(1 + one_ulp / 2 + 2.0 ** -40),
           2.0 ** -133 * 0.5, 2.0 ** -133 * 0.5 + 2.0 ** -170, 2.0 ** -133 * 1.5, 3.4e38, 3.3895e38]
    for x in xs:
        want = _rne_fraction(Fraction(x), 7, -126, 127)
        got = oracle.round_bf16(np.array([x]))[0]
        if isinstance(want, float):
            assert got == want, x
        else:
            assert Fraction(got) == want, x


def test_fp32_rounding_vs_numpy_cast():
    r = np.random.default_rng(3)
    x = r.standard_normal(50000) * np.exp2(r.integers(-150, 120, 50000))
    assert np.array_equal(oracle.f64_to_fp32(x), x.astype(np.float32))


def test_e4m3_encode_matches_torch():
    r = np.random.default_rng(5)
    v = np.concatenate([
        r.uniform(-448, 448, 100000),
        r.standard_normal(50000) * 2.0 ** -8,             # subnormal range
        np.array([464.0 - 1e-9, 2.0 ** -10, 3 * 2.0 ** -11, -2.0 ** -10, 0.0, -0.0, 240 + 8, 240 + 8.0001]),
    ]).astype(np.float32)
    ours = oracle.encode_e4m3(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_rational_ties_to_even_code():
    # midpoints between consecutive positive codes go to the code with an even last bit
    vals = oracle.decode_e4m3(np.arange(0x7F))
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        got = int(oracle.encode_e4m3(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), hex(c)
    with pytest.raises(OverflowError):
        oracle.encode_e4m3(np.array([470.0]))
