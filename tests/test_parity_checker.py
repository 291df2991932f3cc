"""The GPU parity checkers themselves, on the CPU: check_bf16 and check_f32 must accept the
oracle's own result and results within the rule, and must reject planted mistakes of the kinds a
kernel could make (an output two ulps off where no cancellation excuses it, a dropped 128-wide K
chunk, a block exponent off by one, a product with the wrong sign, too many outputs leaning on
the near-cancelling clause, an fp32 value beyond the rounding bound). The rule itself: within one
bf16 ulp of the one-step RNE of the exact sum, or within (K + splits + 17) * 2^-24 * sum|x*w|
plus half an ulp of it for at most clause_cap(n) outputs (fp32 outputs: within the bound)."""
import numpy as np
import pytest

import oracle
import synthetic as S
from parity import check_bf16, check_bf16_exact, check_f32, clause_cap, ordinal


def _case(seed=31, M=6, G=2, N=64, K=512):
    r = S.rng(seed)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 118, 124)
    exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    return x, q, e, exact


def _shift(bits, idx, steps):
    """Move one bf16 pattern `steps` places along the ordinal line (away from zero for steps > 0)."""
    y = np.array(bits, dtype=np.uint16, copy=True)
    v = int(y[idx])
    mag = (v & 0x7FFF) + steps
    y[idx] = (v & 0x8000) | mag
    return y


def _far_from_cancelling(exact, absum):
    """Index of the output whose magnitude is largest relative to sum|x*w| (no cancellation)."""
    return np.unravel_index(np.argmax(np.abs(exact) / absum), exact.shape)


def test_accepts_the_oracle_and_one_ulp():
    x, q, e, exact = _case()
    y = oracle.f64_to_bf16_bits(exact)
    st = check_bf16(y, x, 2, 64, 512, q, e, exact=exact)
    assert st["exact"] == st["n"] and st["by_clause"] == 0
    absum = oracle.abs_products_sum(x, 2, 64, 512, q, e)
    i = _far_from_cancelling(exact, absum)
    for steps in (1, -1):
        st = check_bf16(_shift(y, i, steps), x, 2, 64, 512, q, e, exact=exact)
        assert st["max_ulp"] == 1 and st["by_clause"] == 0


def test_rejects_two_ulps_without_cancellation():
    x, q, e, exact = _case()
    y = oracle.f64_to_bf16_bits(exact)
    absum = oracle.abs_products_sum(x, 2, 64, 512, q, e)
    i = _far_from_cancelling(exact, absum)
    # the clause bound, (K + 81) * 2^-24 * sum|x*w|, is below one ulp of this output
    assert (512 + 81) * 2.0 ** -24 * absum[i] < 2.0 ** -8 * abs(exact[i])
    for steps in (2, -2, 3):
        with pytest.raises(AssertionError, match="fail parity"):
            check_bf16(_shift(y, i, steps), x, 2, 64, 512, q, e, exact=exact)


def test_rejects_a_dropped_chunk():
    M, G, N, K = 6, 2, 64, 512
    x, q, e, exact = _case(M=M, G=G, N=N, K=K)
    x_drop = x.copy()
    x_drop[:, 128:256] = 0                          # group 0 loses its second 128-wide chunk
    y = oracle.gemm(x_drop, G, N, K, q, e)
    with pytest.raises(AssertionError):
        check_bf16(y, x, G, N, K, q, e, exact=exact)
    # the last chunk of the last group only
    x_drop = x.copy()
    x_drop[:, G * K - 128:] = 0
    with pytest.raises(AssertionError):
        check_bf16(oracle.gemm(x_drop, G, N, K, q, e), x, G, N, K, q, e, exact=exact)


def test_rejects_a_block_exponent_off_by_one():
    M, G, N, K = 6, 2, 64, 512
    x, q, e, exact = _case(M=M, G=G, N=N, K=K)
    for delta in (1, -1):
        e_bad = e.copy()
        e_bad[1, 1, 7] = int(e_bad[1, 1, 7]) + delta   # one 32x32 block of group 1, rows 32..63
        with pytest.raises(AssertionError):
            check_bf16(oracle.gemm(x, G, N, K, q, e_bad), x, G, N, K, q, e, exact=exact)
        with pytest.raises(AssertionError):
            check_f32(oracle.gemm(x, G, N, K, q, e_bad, out="f32"), x, G, N, K, q, e, exact=exact)


def test_rejects_one_flipped_product():
    """One weight code with its sign flipped changes each output of its row by 2|x*w| for one
    product: well beyond the bound wherever that product is not tiny."""
    M, G, N, K = 6, 1, 32, 256
    x, q, e, exact = _case(seed=32, M=M, G=G, N=N, K=K)
    X = oracle.bf16_bits_to_f64(x)
    W = oracle.dequant_values(q, e)
    k = int(np.argmax(np.abs(W[0, 5]) * np.abs(X).min(axis=0)))   # a product large in every row
    q_bad = q.copy()
    q_bad[0, 5, k] ^= 0x80
    with pytest.raises(AssertionError):
        check_bf16(oracle.gemm(x, G, N, K, q_bad, e), x, G, N, K, q, e, exact=exact)
    with pytest.raises(AssertionError):
        check_f32(oracle.gemm(x, G, N, K, q_bad, e, out="f32"), x, G, N, K, q, e, exact=exact)


def test_clause_is_capped():
    """Outputs that nearly cancel may sit further than one ulp from the rounded exact sum, within
    the fp32 bound; but only clause_cap(n) of them."""
    n, K = 1000, 4096
    exact = np.full(n, 1e-6)                        # tiny sums of large products
    absum = np.ones(n)
    ref = oracle.f64_to_bf16_bits(exact)
    for n_off, ok in ((clause_cap(n), True), (clause_cap(n) + 1, False)):
        y = ref.copy()
        for i in range(n_off):
            y = _shift(y, i, 3)                     # 3 ulps of 1e-6 is far inside the bound
        if ok:
            st = check_bf16_exact(y, exact, lambda: absum, K)
            assert st["by_clause"] == n_off and st["max_ulp"] == 3
        else:
            with pytest.raises(AssertionError, match="near-cancelling clause"):
                check_bf16_exact(y, exact, lambda: absum, K)
    # beyond the bound itself: rejected whatever the count
    y = ref.copy()
    y[0] = oracle.f64_to_bf16_bits(np.array([1e-6 + 2 * (K + 81) * 2.0 ** -24]))[0]
    with pytest.raises(AssertionError, match="fail parity"):
        check_bf16_exact(y, exact, lambda: absum, K)


def test_f32_accepts_rounding_and_rejects_beyond_the_bound():
    M, G, N, K = 6, 2, 64, 512
    x, q, e, exact = _case(M=M, G=G, N=N, K=K)
    y = oracle.gemm(x, G, N, K, q, e, out="f32")
    check_f32(y, x, G, N, K, q, e, exact=exact)
    absum = oracle.abs_products_sum(x, G, N, K, q, e)
    # a few fp32 ulps anywhere are inside the bound
    y2 = np.nextafter(np.nextafter(y, np.float32(np.inf)), np.float32(np.inf))
    check_f32(y2, x, G, N, K, q, e, exact=exact)
    # one element moved by twice the bound is not
    i = (3, 1, 17)
    y3 = y.copy()
    y3[i] = np.float32(exact[i] + 2 * (K + 81) * 2.0 ** -24 * absum[i])
    with pytest.raises(AssertionError, match="beyond the bound"):
        check_f32(y3, x, G, N, K, q, e, exact=exact)


def test_ordinal_distance_is_monotone():
    """The ulp distance the rule counts: consecutive bf16 patterns are one apart, +0 and -0 are the
    same point, and the smallest subnormals of either sign are one apart from zero."""
    pos = np.arange(0, 0x7F80, dtype=np.uint16)
    o = ordinal(pos)
    assert np.all(np.diff(o) == 1)
    neg = pos | 0x8000
    assert np.all(ordinal(neg) == -o)
    assert ordinal(np.array([0x8000]))[0] == ordinal(np.array([0x0000]))[0] == 0
    assert ordinal(np.array([0x0001]))[0] - ordinal(np.array([0x8001]))[0] == 2
