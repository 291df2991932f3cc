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


def check_bf16(y_bits, x, G, N, K, q, e, exact=None, splits=64):
    """The parity rule for bf16 outputs: every element is within 1 bf16 ulp (ordinal distance) of
    the oracle's one-step RNE of the float64 sum, or (near-cancelling clause) within
    B + half an ulp of the float64 sum, B = budget * 2^-24 * sum|x*w|. Returns stats; raises
    AssertionError on an element that fails both."""
    if exact is None:
        exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    return check_bf16_exact(y_bits, exact, lambda: oracle.abs_products_sum(x, G, N, K, q, e), K, splits)


def check_bf16_exact(y_bits, exact, absum_fn, K, splits=64):
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
