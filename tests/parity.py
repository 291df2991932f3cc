"""Helpers for the GPU parity tests: move seeded inputs to the GPU and compare the library's
outputs with the CPU oracle (test infrastructure; imports the oracle, never the reverse)."""
import numpy as np
import torch

import oracle

U = 2.0 ** -24   # fp32 unit roundoff (round to nearest)


def to_gpu_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def bf16_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordinal(bits):
    """Monotone integer image of bf16 patterns (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def rounding_budget(K, splits=64):
    """Number of fp32 roundings any accumulation order of this library can make per output,
    counted generously: one per product (as if the MFMA summed sequentially), one per wave and
    split partial, plus one."""
    return K + splits + 16 + 1


def clause_cap(n):
    """Most outputs of one check that may pass through the near-cancelling clause: 4 plus one in
    ten thousand. Any fp32 summation order leaves about one output in a hundred thousand more than
    one bf16 ulp away from the exact sum (sums that nearly cancel), so a kernel that needs the
    clause ten times as often has an error of its own, however small each deviation."""
    return 4 + n // 10000


def check_bf16(y_bits, x, G, N, K, q, e, exact=None, splits=64, max_clause=None):
    """The parity rule for bf16 outputs: every element is within 1 bf16 ulp (ordinal distance) of
    the oracle's one-step RNE of the float64 sum, or (near-cancelling clause) within
    B + half an ulp of the float64 sum, B = budget * 2^-24 * sum|x*w|, and at most
    max_clause (default clause_cap(n)) elements use the clause. Returns stats; raises
    AssertionError on an element that fails both, or on too many clause elements."""
    if exact is None:
        exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    return check_bf16_exact(y_bits, exact, lambda: oracle.abs_products_sum(x, G, N, K, q, e), K, splits,
                            max_clause)


def check_bf16_exact(y_bits, exact, absum_fn, K, splits=64, max_clause=None):
    """check_bf16 for a given float64 sum; absum_fn() returns sum|x*w| (computed only when an
    element is more than one ulp away)."""
    ref = oracle.f64_to_bf16_bits(exact)
    y_bits = np.asarray(y_bits, dtype=np.uint16).reshape(ref.shape)
    dist = np.abs(ordinal(y_bits) - ordinal(ref))
    far = dist > 1
    n_clause = 0
    if far.any():
        absum = absum_fn()
        yv = oracle.bf16_bits_to_f64(y_bits)
        # half an ulp of the stored bf16 value
        half_ulp = np.where(yv == 0, 2.0 ** -134,
                            np.ldexp(1.0, np.maximum(np.frexp(np.abs(yv))[1] - 1, -126) - 8))
        bound = rounding_budget(K, splits) * U * absum + half_ulp
        err = np.abs(yv - exact)
        bad = far & ~(err <= bound)
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{int(bad.sum())} outputs fail parity, e.g. at {idx.tolist()}: "
                                 f"gpu {[hex(int(y_bits[tuple(i)])) for i in idx]} "
                                 f"oracle {[hex(int(ref[tuple(i)])) for i in idx]}")
        n_clause = int(far.sum())
        cap = clause_cap(int(ref.size)) if max_clause is None else max_clause
        if n_clause > cap:
            raise AssertionError(f"{n_clause} of {ref.size} outputs need the near-cancelling clause (cap {cap}); "
                                 f"largest distance {int(dist.max())} ulp")
    return dict(n=int(ref.size), within_1ulp=int((dist <= 1).sum()), exact=int((dist == 0).sum()),
                by_clause=n_clause, max_ulp=int(dist.max()) if dist.size else 0)


def check_f32(y, x, G, N, K, q, e, exact=None, splits=64):
    """fp32 outputs: |y - Y_exact| <= budget * 2^-24 * sum|x*w| on every element."""
    if exact is None:
        exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    absum = oracle.abs_products_sum(x, G, N, K, q, e)
    y = np.asarray(y, dtype=np.float64).reshape(exact.shape)
    bound = rounding_budget(K, splits) * U * absum
    err = np.abs(y - exact)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} fp32 outputs beyond the bound, e.g. {idx.tolist()}")
    rel = err / np.maximum(absum, 1e-300)
    return dict(n=int(y.size), max_rel_to_absum=float(rel.max()) if rel.size else 0.0)


# The block-scaled fp8 MFMA sums each group of eight adjacent products inside the instruction in
# a window anchored at the group's largest operand exponents: bits more than 13 places below
# 2^(ea + eb) of the group's largest product are not kept (measured on gfx950 with one-hot and
# two-product inputs). Each of the other seven products of a group then loses less than
# 2^-13 * max|p| of the group, so a group loses less than 2^-10 * sum|p| of the group. Across
# groups, chunks and waves the sums are fp32 additions. Hence, with A = sum_k |x_k w_k|:
#     |y - Y_exact| <= (2^-10 + (K/8 + 32) * 2^-24) * A.
def mx_budget(K):
    return 2.0 ** -10 + (K / 8 + 32) * U


def check_mx_bf16(y_bits, exact, absum, K):
    """bf16 outputs of the fp8 x fp8 GEMM: within 1 bf16 ulp of the one-step RNE of the exact sum,
    or within mx_budget(K) * A + half an ulp of it. Returns stats incl. the largest |err| / A."""
    ref = oracle.f64_to_bf16_bits(exact)
    y_bits = np.asarray(y_bits, dtype=np.uint16).reshape(ref.shape)
    dist = np.abs(ordinal(y_bits) - ordinal(ref))
    yv = oracle.bf16_bits_to_f64(y_bits)
    far = dist > 1
    n_clause = 0
    if far.any():
        half_ulp = np.where(yv == 0, 2.0 ** -134,
                            np.ldexp(1.0, np.maximum(np.frexp(np.abs(yv))[1] - 1, -126) - 8))
        bound = mx_budget(K) * absum + half_ulp
        bad = far & ~(np.abs(yv - exact) <= bound)
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{int(bad.sum())} outputs fail the fp8 parity rule, e.g. at {idx.tolist()}")
        n_clause = int(far.sum())
    return dict(n=int(ref.size), exact=int((dist == 0).sum()), within_1ulp=int((dist <= 1).sum()),
                by_clause=n_clause, max_ulp=int(dist.max()) if dist.size else 0)


def check_mx_f32(y, exact, absum, K):
    """fp32 outputs of the fp8 x fp8 GEMM: |y - Y_exact| <= mx_budget(K) * A everywhere.
    Returns the largest |err| / A (to report how far inside the bound the hardware stays)."""
    y = np.asarray(y, dtype=np.float64).reshape(exact.shape)
    err = np.abs(y - exact)
    bad = ~(err <= mx_budget(K) * absum)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} fp32 outputs beyond the fp8 bound, e.g. {idx.tolist()}")
    rel = err / np.maximum(absum, 1e-300)
    return float(rel.max()) if rel.size else 0.0


# MXFP8 epilogue (fixed-order fp32 sum + MXFP8 quantisation of the output). The GPU quantises its
# own fp32 sums, which differ from RNE_fp32(Y_exact) by at most B = budget * 2^-24 * sum|x*w| per
# output; a code (and a block's scale) may therefore differ from the oracle's ideal epilogue only
# where a value within B of the exact one lies on the other side of a rounding (or binade)
# boundary. Both decisions are monotone in the value, so the check is an interval check.
def _e4m3_sat_codes(t):
    """float64 scaled values -> e4m3 codes: RNE, saturated at +-448 (the quantiser's rule)."""
    F = oracle.formats
    r = F.round_to_binary(t, F.E4M3_FRAC, F.E4M3_EMIN, F.E4M3_EMAX, overflow="inf")
    return F.encode_e4m3(np.clip(r, -F.E4M3_MAX, F.E4M3_MAX))


def e4m3_ordinal(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_mxfp8(yq, ys, exact, absum, K, splits=64):
    """yq [M, L], ys [M, L/32] from the GPU; exact and absum [M, L] float64. Returns stats."""
    import oracle.epilogue as EP
    import oracle.mx as MX
    M, L = exact.shape
    yq = np.asarray(yq, dtype=np.uint8).reshape(M, L)
    ys = np.asarray(ys, dtype=np.uint8).reshape(M, L // 32)
    iq, iscale = EP.quantize_mx_f32(oracle.f64_to_fp32(exact))
    B = rounding_budget(K, splits) * U * absum
    nb = L // 32
    amax = np.abs(exact).reshape(M, nb, 32).max(axis=2)
    bmax = B.reshape(M, nb, 32).max(axis=2)
    s_lo = MX.mx_scale_exponent(np.maximum(amax - bmax, 0.0))
    s_hi = MX.mx_scale_exponent(amax + bmax)
    sg = ys.astype(np.int64) - 127
    scale_ok = (ys == iscale) | ((sg >= s_lo) & (sg <= s_hi) & (ys != 255))
    if not scale_ok.all():
        idx = np.argwhere(~scale_ok)[:5]
        raise AssertionError(f"{int((~scale_ok).sum())} block scales out of range, e.g. {idx.tolist()}: "
                             f"gpu {[int(ys[tuple(i)]) for i in idx]} ideal {[int(iscale[tuple(i)]) for i in idx]}")
    sgk = np.repeat(sg, 32, axis=1)
    same = (yq == iq) & np.repeat(ys == iscale, 32, axis=1)
    lo = e4m3_ordinal(_e4m3_sat_codes(np.ldexp(exact - B, -sgk)))
    hi = e4m3_ordinal(_e4m3_sat_codes(np.ldexp(exact + B, -sgk)))
    o = e4m3_ordinal(yq)
    ok = same | ((o >= lo) & (o <= hi))
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{int((~ok).sum())} codes fail the epilogue rule, e.g. {idx.tolist()}: "
                             f"gpu {[hex(int(yq[tuple(i)])) for i in idx]} ideal {[hex(int(iq[tuple(i)])) for i in idx]}")
    return dict(n=int(yq.size), same=int(same.sum()), by_clause=int((~same).sum()),
                blocks=int(ys.size), scale_differs=int((ys != iscale).sum()))
