"""Planted mistakes in the oracle, on the CPU. Each case below patches one plausible slip into one
oracle function - a wrong exponent bias, a wrong subnormal quantum, an off-by-one block factor or
block exponent, ties rounded away from zero, a double rounding, a swapped group, a dropped term,
a transposed tile, a missing MX offset, the wrong largest e4m3 value, a lost pad exponent, a
scale check that lets +inf through, a swapped summation order, exponents of the wrong row, an
output rounded before it is quantised - and requires that at least one of the pins guarding that
function fails. This checks the pins, not the oracle; pytest's monkeypatch restores the oracle
after each case."""
import itertools
import math

import numpy as np
import pytest

import oracle
import oracle.epilogue as EP
import oracle.formats as F
import oracle.mx as MX
import oracle.ops as OPS
import oracle.row32 as R32

import test_oracle_epilogue as TE
import test_oracle_formats as TF
import test_oracle_gemm as TG
import test_oracle_mx as TM
import test_oracle_row32 as TR
import test_oracle_twin as TT


def _calls(fn):
    """Keyword arguments of every parametrised instance of a pin (one empty call if none)."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    grids = []
    for m in marks:
        names = [n.strip() for n in m.args[0].split(",")]
        grids.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in m.args[1]])
    for combo in itertools.product(*grids):
        kw = {}
        for d in combo:
            kw.update(d)
        yield kw


def _first_failing_pin(pins):
    for fn in pins:
        for kw in _calls(fn):
            try:
                fn(**kw)
            except (Exception, pytest.fail.Exception):   # an assertion, pytest.raises not met,
                return fn.__name__                         # or the mutant breaking an invariant
    return None


def _e4m3_table(bias=7, sub_quantum=-9):
    vals = []
    for c in range(256):
        s, E, m = c >> 7, (c >> 3) & 15, c & 7
        if E == 15 and m == 7:
            vals.append(math.nan)
            continue
        mag = m * 2.0 ** sub_quantum if E == 0 else (1 + m / 8) * 2.0 ** (E - bias)
        vals.append(-mag if s else mag)
    return np.array(vals, dtype=np.float64)


# --- mutants: each takes pytest's monkeypatch and installs one mistake ---------------------------
def m_e4m3_bias_8(mp):
    mp.setattr(F, "E4M3_TABLE", _e4m3_table(bias=8))


def m_e4m3_subnormal_quantum(mp):
    mp.setattr(F, "E4M3_TABLE", _e4m3_table(sub_quantum=-10))


def m_block_factor_off_by_one(mp):
    mp.setattr(F, "exp_factor", lambda b: np.ldexp(1.0, np.asarray(b).astype(np.int64) - 126))


def m_ties_away_from_zero(mp):
    orig = F.round_to_binary

    def rtb(x, frac_bits, emin, emax, overflow="inf"):
        x = np.asarray(x, dtype=np.float64)
        mag = np.abs(x)
        finite = np.isfinite(mag)
        safe = np.where(finite, mag, 0.0)
        _, e2 = np.frexp(safe)
        q = np.maximum(e2.astype(np.int64) - 1, emin) - frac_bits
        r = np.ldexp(np.floor(np.ldexp(safe, -q) + 0.5), q)       # half away from zero
        largest = (2.0 - 2.0 ** -frac_bits) * 2.0 ** emax
        if overflow == "raise" and np.any((r > largest) & finite):
            raise OverflowError
        r = np.where(r > largest, np.inf, r)
        return np.copysign(np.where(finite, r, mag), x)
    assert orig is not rtb
    mp.setattr(F, "round_to_binary", rtb)


def m_double_rounding_through_fp32(mp):
    orig = F.round_bf16
    twice = lambda x: orig(F.round_fp32(x))
    mp.setattr(F, "round_bf16", twice)
    mp.setattr(oracle, "round_bf16", twice)


def _patched_gemm(transform):
    def gemm_exact_f64(x_bits, G, N, K, q, e):
        q = np.asarray(q, dtype=np.uint8)
        if np.isin(q, F.E4M3_NAN_CODES).any():
            raise ValueError("NaN weight code")
        x_bits = np.asarray(x_bits, dtype=np.uint16)
        M = x_bits.shape[0]
        X = F.bf16_bits_to_f64(x_bits[:, : G * K]).reshape(M, G, K)
        W = OPS.dequant_values(q, e)
        return transform(X, W, M, G, N, K)
    return gemm_exact_f64


def m_swapped_groups(mp):
    def t(X, W, M, G, N, K):
        return np.stack([X[:, (g + 1) % G, :] @ W[g].T for g in range(G)], axis=1)
    mp.setattr(OPS, "gemm_exact_f64", _patched_gemm(t))


def m_dropped_last_term(mp):
    def t(X, W, M, G, N, K):
        return np.stack([X[:, g, : K - 1] @ W[g][:, : K - 1].T for g in range(G)], axis=1)
    mp.setattr(OPS, "gemm_exact_f64", _patched_gemm(t))


def m_transposed_tile(mp):
    orig = OPS.dequant_values

    def dq(q, e):
        W = orig(q, e)
        G, N, K = W.shape
        return W.reshape(G, N // 32, 32, K // 32, 32).transpose(0, 1, 4, 3, 2).reshape(G, N, K)
    mp.setattr(OPS, "dequant_values", dq)


def m_block_exponent_too_small(mp):
    orig = OPS.block_exponent
    mp.setattr(OPS, "block_exponent", lambda a: np.clip(orig(a) - 1, -127, 127))


def m_block_exponent_too_large(mp):
    orig = OPS.block_exponent
    mp.setattr(OPS, "block_exponent", lambda a: np.clip(orig(a) + 1, -127, 127))


def m_mx_offset_missing(mp):
    orig = MX.mx_scale_exponent
    mp.setattr(MX, "mx_scale_exponent", lambda a: np.clip(orig(a) + 8, -127, 127))


def m_e4m3_largest_480(mp):
    mp.setattr(F, "E4M3_MAX", 480.0)


def m_pad_exponent_zero(mp):
    mp.setattr(OPS, "PAD_EXPONENT", 0)


def m_scales_accept_inf(mp):
    def scales_from_f32(s, N=None, K=None):
        s = np.asarray(s)
        if s.dtype != np.float32:
            raise OPS.ScaleError("scales must be float32")
        if N is not None and K is not None and s.shape != (N // 32, K // 32):
            raise OPS.ScaleError("shape")
        bits = s.view(np.uint32)
        good = ((bits & 0x7FFFFF) == 0) & ((bits >> 31) == 0) & (((bits >> 23) & 0xFF) >= 1)
        if not np.all(good):
            raise OPS.ScaleError("refused")
        return ((bits >> 23) & 0xFF).astype(np.uint8)
    mp.setattr(OPS, "scales_from_f32", scales_from_f32)
    mp.setattr(oracle, "scales_from_f32", scales_from_f32)


def m_epilogue_order_ignored(mp):
    orig = EP._sum
    mp.setattr(EP, "_sum", lambda part, S, order: orig(part, S, EP.ORDER_ASCENDING))


def m_row_exponents_of_the_neighbour_row(mp):
    orig = R32.expand_row_exponents

    def ex(e, K):
        f = orig(e, K)
        return f[:, np.arange(f.shape[1]) ^ 1, :]
    mp.setattr(R32, "expand_row_exponents", ex)


def m_epilogue_quantises_bf16(mp):
    def ideal(x_bits, G, N, K, q, e):
        Y = OPS.gemm_exact_f64(x_bits, G, N, K, q, e)
        M = Y.shape[0]
        c, s = EP.quantize_mx_f32(F.round_bf16(Y).astype(np.float32).reshape(M, G * N))
        return c, s, Y
    mp.setattr(EP, "gemm_mxfp8_ideal", ideal)


CASES = [
    (m_e4m3_bias_8, [TF.test_e4m3_decode_matches_torch_for_all_codes, TF.test_e4m3_landmarks_golden]),
    (m_e4m3_subnormal_quantum, [TF.test_e4m3_decode_matches_torch_for_all_codes, TF.test_e4m3_landmarks_golden]),
    (m_block_factor_off_by_one, [TF.test_exp_factor_closed_form, TG.test_gemm_equals_exact_rational_brute_force,
                                 TG.test_dequant_equals_rational_brute_force_all_codes_all_exponents]),
    (m_ties_away_from_zero, [TF.test_bf16_rounding_matches_torch_on_fp32_values,
                             TF.test_bf16_rounding_one_step_from_f64_vs_rational_brute_force,
                             TF.test_e4m3_encode_rational_ties_to_even_code]),
    (m_double_rounding_through_fp32, [TF.test_bf16_rounding_one_step_from_f64_vs_rational_brute_force,
                                      TG.test_gemm_equals_exact_rational_brute_force]),
    (m_swapped_groups, [TG.test_gemm_equals_exact_rational_brute_force, TG.test_one_hot_rows_select_single_weights]),
    (m_dropped_last_term, [TG.test_gemm_equals_exact_rational_brute_force,
                           TG.test_integer_exact_regime_matches_integer_matmul]),
    (m_transposed_tile, [TG.test_gemm_equals_exact_rational_brute_force, TG.test_one_hot_rows_select_single_weights]),
    (m_block_exponent_too_small, [TT.test_worked_block_exponents_golden,
                                  TT.test_block_exponent_integer_rule_for_every_bf16_magnitude]),
    (m_block_exponent_too_large, [TT.test_worked_block_exponents_golden,
                                  TT.test_block_exponent_integer_rule_for_every_bf16_magnitude]),
    (m_mx_offset_missing, [TM.test_scale_exponent_integer_rule_over_every_bf16_magnitude, TM.test_worked_blocks]),
    (m_e4m3_largest_480, [TM.test_worked_blocks, TT.test_worked_block_exponents_golden]),
    (m_pad_exponent_zero, [TG.test_pad_k_is_bitwise_invariant]),
    (m_scales_accept_inf, [TG.test_scales_golden]),
    (m_epilogue_order_ignored, [TE.test_order_decides_worked_cases, TE.test_sums_match_exact_rationals_step_by_step]),
    (m_row_exponents_of_the_neighbour_row, [TR.test_gemm_equals_exact_rational_brute_force]),
    (m_epilogue_quantises_bf16, [TE.test_ideal_epilogue_against_rational_brute_force]),
]


@pytest.mark.parametrize("mutant,pins", CASES, ids=[c[0].__name__[2:] for c in CASES])
def test_a_planted_mistake_fails_a_pin(monkeypatch, mutant, pins):
    with monkeypatch.context() as mp:
        mutant(mp)
        failed = _first_failing_pin(pins)
    assert failed is not None, f"no pin caught {mutant.__name__}"
