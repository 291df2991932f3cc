"""GPU parity on seeded random shapes, through the C ABI: every GEMM entry point (bf16 and fp32
output, explicit splits, the MXFP8 output epilogue, the fp8 x fp8 path, the row-scale twin) on
shapes drawn from the whole accepted range - 1..256 rows, 1..3 groups, N and K any multiple of 32
(K whole 128-chunks where an entry point requires it), odd exponent ranges, strided activations -
against the oracle under the same parity rules as the fixed-shape tests. Sizes are capped so that
the float64 oracle stays quick."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import oracle.mx as MX
import oracle.row32 as R32
import synthetic as S
from parity import (bf16_bits, check_bf16, check_bf16_exact, check_f32, check_mx_bf16, check_mxfp8, to_gpu_bf16,
                    to_gpu_u8)

pytestmark = pytest.mark.gpu

N_CASES = 24


def _shape(r, k128=False, max_m=256):
    while True:
        M = int(r.choice([1, 2, 3, 5, 6, 8, 9, 13, 16, 17, 31, 33, 47, 64, 65, 100, 128, 129, 192, 200, 256]))
        M = min(M, max_m)
        G = int(r.integers(1, 4))
        N = 32 * int(r.integers(1, 48))
        K = (128 if k128 else 32) * int(r.integers(1, 33 if k128 else 129))
        if M * G * N * K <= 60_000_000:
            return M, G, N, K


def _inputs(r, M, G, N, K, row_exps=False):
    lo = int(r.integers(100, 125))
    hi = lo + int(r.integers(0, 12))
    pad = 8 * int(r.integers(0, 3))                  # ldx = G*K + pad
    x = S.bf16_normal(r, (M, G * K + pad), scale=float(2.0 ** r.integers(-4, 4)))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N, K // 32) if row_exps else (G, N // 32, K // 32), lo, hi)
    return x, q, e


def _x_gpu(x, G, K):
    """bf16 activations on the GPU with their row stride (a view of the padded rows)."""
    return to_gpu_bf16(x)[:, : G * K]


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_gemm_bf16_f32_and_splits(case):
    r = S.rng(12000 + case)
    M, G, N, K = _shape(r)
    x, q, e = _inputs(r, M, G, N, K)
    split = int(r.choice([0, 0, 1, 2, 3, 5]))
    plan = B.bsfp8_plan_info(M, G, N, K, split_k=split)
    print(f"case {case}: M={M} G={G} N={N} K={K} split={split} plan {plan}", flush=True)
    xt, qt, et = _x_gpu(x, G, K), to_gpu_u8(q), to_gpu_u8(e)
    y = B.bsfp8_gemm(xt, qt, et, split_k=split)
    y32 = B.bsfp8_gemm(xt, qt, et, split_k=split, out_dtype="f32")
    torch.cuda.synchronize()
    exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    st = check_bf16(bf16_bits(y), x, G, N, K, q, e, exact=exact)
    check_f32(y32.cpu().numpy(), x, G, N, K, q, e, exact=exact)
    # the bf16 result is the RNE of the same fp32 sums
    assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    print(st, flush=True)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_gemm_mxfp8(case):
    r = S.rng(13000 + case)
    M, G, N, K = _shape(r)
    x, q, e = _inputs(r, M, G, N, K)
    split = int(r.choice([0, 0, 0, 1, 2]))
    plan = B.bsfp8_plan_info(M, G, N, K, split_k=split, path=3)
    print(f"case {case}: M={M} G={G} N={N} K={K} split={split} plan {plan}", flush=True)
    xt, qt, et = _x_gpu(x, G, K), to_gpu_u8(q), to_gpu_u8(e)
    yq, ys = B.bsfp8_gemm_mxfp8(xt, qt, et, split_k=split)
    y32 = B.bsfp8_gemm_config(xt, qt, et, plan["cfg"], plan["cps"], out_dtype="f32")   # the same plan
    q2, s2 = B.bsfp8_reduce_quantize_mx(y32.reshape(1, M, G * N), B.SUM_ASCENDING)
    torch.cuda.synchronize()
    assert torch.equal(yq, q2) and torch.equal(ys, s2)
    exact = oracle.gemm_exact_f64(x, G, N, K, q, e).reshape(M, G * N)
    absum = oracle.abs_products_sum(x, G, N, K, q, e).reshape(M, G * N)
    print(check_mxfp8(yq.cpu().numpy(), ys.cpu().numpy(), exact, absum, K, plan["splits"]), flush=True)


@pytest.mark.parametrize("case", range(12))
def test_random_gemm_mx(case):
    r = S.rng(14000 + case)
    M, G, N, K = _shape(r, k128=True)
    x, q, e = _inputs(r, M, G, N, K)
    print(f"case {case}: M={M} G={G} N={N} K={K} cfg {B.bsfp8_mx_plan(M, G, N)}", flush=True)
    xq, xs = MX.quantize_mx(x, G * K)
    gq, gs = B.bsfp8_quantize_mx(_x_gpu(x, G, K))
    y = B.bsfp8_gemm_mx(gq, gs, to_gpu_u8(q), to_gpu_u8(e))
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), xq) and np.array_equal(gs.cpu().numpy(), xs)
    exact = MX.gemm_mx_exact_f64(xq, xs, G, N, K, q, e)
    absum = MX.abs_products_sum_mx(xq, xs, G, N, K, q, e)
    print(check_mx_bf16(bf16_bits(y), exact, absum, K), flush=True)


@pytest.mark.parametrize("case", range(12))
def test_random_gemm_row32(case):
    r = S.rng(15000 + case)
    M, G, N, K = _shape(r, k128=True, max_m=16)
    x, q, e = _inputs(r, M, G, N, K, row_exps=True)
    print(f"case {case}: M={M} G={G} N={N} K={K}", flush=True)
    y = B.bsfp8_gemm_row32(_x_gpu(x, G, K), to_gpu_u8(q), to_gpu_u8(e))
    torch.cuda.synchronize()
    exact = R32.gemm_exact_f64_row32(x, G, N, K, q, e)
    print(check_bf16_exact(bf16_bits(y), exact, lambda: R32.abs_products_sum_row32(x, G, N, K, q, e), K), flush=True)
