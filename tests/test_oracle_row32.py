"""Pins of the per-(row, 32-column) scale oracle (oracle/row32.py), CPU only: equality with the
pinned 32x32 oracle where the two formats coincide (exponents shared by the 32 rows of a block;
one real row padded into a 32x32 block with zero rows), an exact rational brute force of the GEMM,
round trips, exact rejection of perturbed blocks, and a block that only the finer format can
represent."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.row32 as R
import synthetic as S
from test_oracle_gemm import _bf16_fraction, _e4m3_fraction, _rne_bf16_bits


def _row_exponents(r, G, N, K, lo=110, hi=135):
    return S.exponent_bytes(r, (G, N, K // 32), lo, hi)


def test_dequant_and_gemm_equal_the_32x32_oracle_on_shared_exponents():
    r = S.rng(9000)
    G, N, K, M = 2, 64, 256, 5
    q = S.e4m3_codes(r, (G, N, K))
    e32 = S.exponent_bytes(r, (G, N // 32, K // 32), 100, 140)
    e_rows = np.repeat(e32, 32, axis=1)                    # every row of a block: the block's byte
    assert np.array_equal(R.dequant_bf16_row32(q, e_rows), oracle.dequant_bf16(q, e32))
    x = S.bf16_normal(r, (M, G * K))
    for out in ("bf16", "f32"):
        assert np.array_equal(R.gemm_row32(x, G, N, K, q, e_rows, out=out),
                              oracle.gemm(x, G, N, K, q, e32, out=out))


def test_gemm_equals_exact_rational_brute_force():
    r = S.rng(9001)
    G, N, K, M = 2, 8, 64, 2
    q = S.e4m3_codes(r, (G, N, K))
    e = _row_exponents(r, G, N, K, 0, 246)                 # incl. exponents far from 127
    e[0, 0, 0] = 0                                         # (246: 448 * 2^119 is still a finite bf16)
    e[1, 3, 1] = 246
    x = S.bf16_normal(r, (M, G * K))
    got = R.gemm_row32(x, G, N, K, q, e)
    for m in range(M):
        for g in range(G):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    w = _e4m3_fraction(int(q[g, n, k])) * Fraction(2) ** (int(e[g, n, k // 32]) - 127)
                    acc += _bf16_fraction(int(x[m, g * K + k])) * _bf16_fraction(_rne_bf16_bits(w))
                assert got[m, g, n] == _rne_bf16_bits(acc), (m, g, n)


def test_twin_equals_the_32x32_twin_of_a_row_padded_with_zero_rows():
    # a 1x32 block and a 32x32 block made of that row and 31 zero rows have the same amax, so the
    # same exponent, codes (zeros encode to zero and rebuild exactly) and verdict
    r = S.rng(9002)
    G, N, K = 1, 6, 96
    src_q = S.e4m3_codes(r, (G, N, K))
    src_e = _row_exponents(r, G, N, K, 115, 125)
    w = R.dequant_bf16_row32(src_q, src_e)
    w[0, 2, 40] ^= 1                                       # a perturbed, non-exact block
    w[0, 4, 0:32] = 0                                      # an all-zero block
    t = R.make_twin_row32(w)
    for n in range(N):
        pad = np.zeros((G, 32, K), dtype=np.uint16)
        pad[:, 0, :] = w[:, n, :]
        ref = oracle.make_twin(pad)
        assert np.array_equal(t.q[:, n, :], ref.q[:, 0, :]), n
        assert np.array_equal(t.e[:, n, :], ref.e[:, 0, :]), n
        assert np.array_equal(t.ok[:, n, :], ref.ok[:, 0, :]), n
    assert not t.accepted and t.ok[0, 2, 1] == 0 and t.ok.sum() == N * K // 32 - 1


def test_round_trip_and_exact_rejection():
    r = S.rng(9003)
    G, N, K = 2, 32, 256
    q = S.e4m3_codes(r, (G, N, K))
    e = _row_exponents(r, G, N, K, 115, 125)
    w = R.dequant_bf16_row32(q, e)
    t = R.make_twin_row32(w)
    assert t.accepted
    assert np.array_equal(R.dequant_bf16_row32(t.q, t.e), w)
    # +1 on the bf16 pattern of one nonzero element in a tenth of the blocks: exactly those reject
    wp = w.copy()
    blocks = np.argwhere(r.random((G, N, K // 32)) < 0.1)
    for g, n, b in blocks:
        nz = np.flatnonzero(wp[g, n, 32 * b: 32 * b + 32] & 0x7FFF)
        wp[g, n, 32 * b + nz[0]] += 1
    tp = R.make_twin_row32(wp)
    want = np.ones((G, N, K // 32), dtype=np.uint8)
    want[tuple(blocks.T)] = 0
    assert np.array_equal(tp.ok, want) and not tp.accepted


def test_the_finer_grid_represents_what_a_32x32_block_cannot():
    # two rows of one 32x32 block whose magnitudes differ by 2^16: the shared block exponent
    # leaves the small row's values below e4m3's resolution, a per-row exponent does not
    small = oracle.f64_to_bf16_bits(np.array([1.0 + i / 8 for i in range(8)] * 4) * 2.0 ** -14)
    big = oracle.f64_to_bf16_bits(np.full(32, 448.0) * 2.0 ** 2)
    w = np.zeros((1, 32, 32), dtype=np.uint16)
    w[0, 0] = big
    w[0, 1] = small
    assert not oracle.make_twin(w).accepted
    t = R.make_twin_row32(w)
    assert t.accepted
    # 448 * 2^-22 = 1.75 * 2^-14 < 1.875 * 2^-14 <= 448 * 2^-21: the small row's exponent is -21
    assert t.e[0, 0, 0] == 127 + 2 and t.e[0, 1, 0] == 127 - 21
    assert np.array_equal(R.dequant_bf16_row32(t.q, t.e), w)


def test_non_finite_blocks():
    w = np.zeros((1, 2, 64), dtype=np.uint16)
    w[0, 0, 3] = 0x7F80
    w[0, 1, 40] = 0xFFC1
    t = R.make_twin_row32(w)
    assert t.e[0, 0, 0] == 255 and t.ok[0, 0, 0] == 0 and (t.q[0, 0, :32] == 0x7F).all()
    assert t.e[0, 1, 1] == 255 and t.ok[0, 1, 1] == 0
    assert t.ok[0, 0, 1] == 1 and t.ok[0, 1, 0] == 1 and t.e[0, 0, 1] == 0   # zero blocks: byte 0
