"""Pins of the oracle twin encoder (make_twin of the wo_a_w8.py page) on the CPU: worked blocks,
an exact integer rule for the block exponent over every bf16 magnitude, a brute force over all
block exponents, the round trip, and rejection of perturbed blocks."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _block_with_amax(amax, fill=0.0):
    """One 32x32 bf16 block whose largest magnitude is `amax` (must be bf16-exact)."""
    v = np.full((1, 32, 32), fill)
    v[0, 5, 7] = amax
    return oracle.f64_to_bf16_bits(v)


def test_worked_block_exponents_golden():
    with open(os.path.join(GOLDEN, "twin_blocks.txt")) as f:
        rows = [ln.split("#", 1)[0].split() for ln in f if ln.split("#", 1)[0].strip()]
    for amax, byte in rows:
        assert int(oracle.block_exponent(np.array([float(amax)]))[0]) + 127 == int(byte), amax
        if float(amax) == float(oracle.round_bf16(np.array([float(amax)]))[0]):
            t = oracle.make_twin(_block_with_amax(float(amax)))
            assert int(t.e[0, 0, 0]) == int(byte), amax


def test_block_exponent_integer_rule_for_every_bf16_magnitude():
    # every positive finite bf16 pattern a: the exponent must be the least integer e with
    # max(a, 2^-126) <= 7 * 2^(6 + e), decided here with integers only
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    a = oracle.bf16_bits_to_f64(bits)
    got = oracle.block_exponent(a)
    for b, ge in zip(bits.tolist()[::7], got.tolist()[::7]):
        ef, m = b >> 7, b & 0x7F
        # a' = max(a, 2^-126) as integer mantissa * 2^p
        if ef == 0:
            mant, p = 1, -126                         # subnormals are clamped up to 2^-126
        else:
            mant, p = 128 + m, ef - 127 - 7
        e = -200
        while Fraction(mant) * Fraction(2) ** p > 7 * Fraction(2) ** (6 + e):
            e += 1
        assert ge == max(-127, min(127, e)), hex(b)


def _representable_at(vals, e):
    """True when every value is exactly an e4m3 value times 2^e (brute force)."""
    table = set(Fraction(float(v)) for v in oracle.decode_e4m3(np.arange(256)) if np.isfinite(v))
    return all(Fraction(float(v)) / Fraction(2) ** e in table for v in vals)


def test_accept_iff_some_exponent_represents_the_block_brute_force():
    r = S.rng(99)
    for trial in range(24):
        # small tiles inside one 32x32 block; the rest of the block is zero
        e0 = int(r.integers(-20, 10))
        codes = S.e4m3_codes(r, 6)
        vals = oracle.decode_e4m3(codes) * 2.0 ** e0
        if trial % 3 == 1:
            vals[2] = vals[2] * (1 + 2.0 ** -7)       # one more significant bit: never representable
        if trial % 3 == 2:
            vals[3] = vals[3] * 2.0 ** -9            # wider spread: maybe not representable
        blk = np.zeros((1, 32, 32))
        blk[0, 0, :6] = vals
        w = oracle.f64_to_bf16_bits(blk)
        wv = oracle.bf16_bits_to_f64(w)[0, 0, :6]
        any_e = any(_representable_at(wv, e) for e in range(-127, 128))
        t = oracle.make_twin(w)
        assert bool(t.ok[0, 0, 0]) == any_e, trial
        if any_e:
            # the chosen (least) exponent is itself one that works
            assert _representable_at(wv, int(t.e[0, 0, 0]) - 127)


def test_round_trip_of_exact_weights_is_accepted_and_bit_identical():
    src = S.twin_source(4000, G=2, R=64, D=128)
    w = oracle.dequant_bf16(src["q"], src["e"])
    t = oracle.make_twin(w)
    assert t.accepted and t.ok.all()
    assert np.array_equal(oracle.dequant_bf16(t.q, t.e), w)
    # the encoded exponent never exceeds the generating one, and equals it when the block's
    # largest code magnitude exceeds 224 (a block whose codes stay at or below 224 = 448 / 2 fits
    # one exponent lower)
    assert np.all(t.e <= src["e"])


def test_perturbed_blocks_are_rejected_exactly():
    src = S.twin_source(4001, G=1, R=128, D=256)
    w = oracle.dequant_bf16(src["q"], src["e"])
    wp, mask = S.perturb_one_element(w, S.rng(4002), 0.1)
    assert mask.any()
    t = oracle.make_twin(wp)
    assert not t.accepted
    assert np.array_equal(t.ok.astype(bool), ~mask)


def test_zero_block_and_signed_zero():
    w = np.zeros((1, 32, 64), dtype=np.uint16)
    w[0, 3, 40] = 0x8000                              # -0 in the second block
    t = oracle.make_twin(w)
    assert t.accepted
    assert t.e.tolist() == [[[0, 0]]]
    assert t.q[0, 3, 40] == 0x80 and np.count_nonzero(t.q) == 1


def test_extra_bit_rejected_and_non_finite_block_marked():
    w = _block_with_amax(1.0, fill=0.5)
    w[0, 0, 0] = 0x3F81                               # 1 + 2^-7: 8 significant bits
    t = oracle.make_twin(w)
    assert not t.accepted
    w2 = np.concatenate([_block_with_amax(2.0), _block_with_amax(2.0)], axis=2)
    w2[0, 1, 33] = 0x7F80                             # +inf in block 1
    t2 = oracle.make_twin(w2)
    assert t2.ok.tolist() == [[[1, 0]]]
    assert t2.e[0, 0, 1] == 255 and np.all(t2.q[0, :, 32:] == 0x7F)


def test_bf16_subnormal_block_round_trips():
    w = np.zeros((1, 32, 32), dtype=np.uint16)
    w[0, 0, 0] = 0x0001                               # 2^-133, the smallest bf16 subnormal
    w[0, 1, 1] = 0x8003                               # -3 * 2^-133
    t = oracle.make_twin(w)
    assert t.accepted and t.e[0, 0, 0] == 0
    assert np.array_equal(oracle.dequant_bf16(t.q, t.e), w)


@pytest.mark.parametrize("e_gen", [-12, -4, 0, 20])
def test_exponent_recovered_when_block_holds_a_large_code(e_gen):
    r = S.rng(50 + e_gen)
    q = S.e4m3_codes(r, (1, 32, 32))
    q[0, 0, 0] = 0x7E                                 # 448 present: the exponent is recovered
    e = np.full((1, 1, 1), e_gen + 127, dtype=np.uint8)
    w = oracle.dequant_bf16(q, e)
    t = oracle.make_twin(w)
    assert t.accepted and int(t.e[0, 0, 0]) == e_gen + 127
    assert np.array_equal(t.q[(q & 0x7F) != 0], q[(q & 0x7F) != 0])
