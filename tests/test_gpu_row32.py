"""GPU parity of the per-(row, 32-column) scale path (twin encoder and GEMM) against the CPU oracle
(oracle/row32.py), through the C ABI. Twin bytes must match bit for bit; GEMM outputs follow the
bf16 path's parity rule (parity.check_bf16_exact)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import oracle.row32 as R
import synthetic as S
from parity import bf16_bits, check_bf16_exact, check_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _twin_gpu(w_bits):
    t = B.bsfp8_make_twin_row32(to_gpu_bf16(w_bits))
    torch.cuda.synchronize()
    return t.accepted, t.q.cpu().numpy(), t.e.cpu().numpy(), t.ok.cpu().numpy(), t.n_bad


def test_make_twin_row32_exact_perturbed_and_edge_blocks_bitwise():
    r = S.rng(9100)
    G, N, K = 2, 96, 512
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N, K // 32), 105, 135)
    w = R.dequant_bf16_row32(q, e)
    acc, gq, ge, gok, nbad = _twin_gpu(w)
    ref = R.make_twin_row32(w)
    assert acc and ref.accepted and nbad == 0
    assert np.array_equal(gq, ref.q) and np.array_equal(ge, ref.e) and np.array_equal(gok, ref.ok)
    # perturbed blocks, random bf16 weights, zero / subnormal / non-finite blocks
    wp = w.copy()
    wp[0, 3, 70] += 1
    wp[1, 50, 0:32] = 0
    wp[1, 51, 32:64] = np.arange(1, 33, dtype=np.uint16)
    wp[1, 52, 64] = 0x7F80
    wp[0, 9, 500] = 0xFFC1
    for ww in (wp, S.bf16_normal(r, (G, N, K), scale=0.02)):
        acc, gq, ge, gok, nbad = _twin_gpu(ww)
        ref = R.make_twin_row32(ww)
        assert acc == ref.accepted and nbad == int((ref.ok == 0).sum())
        assert np.array_equal(gq, ref.q) and np.array_equal(ge, ref.e) and np.array_equal(gok, ref.ok)


def test_make_twin_row32_every_bf16_magnitude_as_a_block_amax():
    mags = np.arange(0, 0x7F80, dtype=np.uint16)
    n = len(mags)
    w = np.zeros((1, n, 32), dtype=np.uint16)
    w[0, :, 0] = mags                                     # the block's amax and only nonzero value
    w[0, :, 1] = mags // 3                                # a smaller companion
    w[0, 1::2, 0] |= 0x8000
    w = w.reshape(1, n // 8, 256) if n % 8 == 0 else w
    acc, gq, ge, gok, nbad = _twin_gpu(w)
    ref = R.make_twin_row32(w)
    assert np.array_equal(gq, ref.q) and np.array_equal(ge, ref.e) and np.array_equal(gok, ref.ok)


def _inputs(seed, M, G, N, K, elo=110, ehi=130):
    r = S.rng(seed)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N, K // 32), elo, ehi)
    return x, q, e


def _check(y, x, G, N, K, q, e):
    exact = R.gemm_exact_f64_row32(x, G, N, K, q, e)
    return check_bf16_exact(bf16_bits(y), exact, lambda: R.abs_products_sum_row32(x, G, N, K, q, e), K)


@pytest.mark.parametrize("M,G,N,K", [(1, 1, 32, 128), (6, 2, 64, 1024), (8, 1, 96, 4096), (11, 1, 64, 640),
                                     (16, 1, 1280, 5120), (3, 4, 32, 8192)])
def test_gemm_row32_parity(M, G, N, K):
    x, q, e = _inputs(9200 + M + K, M, G, N, K)
    y = B.bsfp8_gemm_row32(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e))
    torch.cuda.synchronize()
    st = _check(y, x, G, N, K, q, e)
    print(f"M={M} G={G} N={N} K={K}: {st}")


def test_every_row_scale_configuration_and_split():
    G, N, K = 2, 64, 1024
    for cfg in range(B.bsfp8_num_configs()):
        info = B.bsfp8_config_info(cfg)
        if not info["row_scales"]:
            continue
        M = min(2 * info["BM"] - 3, 16)
        x, q, e = _inputs(9300 + cfg, M, G, N, K)
        for cps in sorted({1, 3, info["CW"] * info["NWK"]}):
            print(f"row-scale cfg {cfg} {info} cps {cps} M {M}", flush=True)
            y = B.bsfp8_gemm_row32_config(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e), cfg, cps)
            torch.cuda.synchronize()
            _check(y, x, G, N, K, q, e)
            yf = B.bsfp8_gemm_row32_config(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e), cfg, cps, out_dtype="f32")
            torch.cuda.synchronize()
            exact = R.gemm_exact_f64_row32(x, G, N, K, q, e)
            absum = R.abs_products_sum_row32(x, G, N, K, q, e)
            err = np.abs(yf.cpu().numpy().astype(np.float64) - exact)
            assert (err <= (K + 64 + 17) * 2.0 ** -24 * absum).all()


def test_row_exponents_shared_by_a_block_match_the_32x32_gemm_bitwise():
    # replicating each 32x32 exponent over its 32 rows gives the same weights, and the row-scale
    # plan uses the same waves and chunks as the 32x32 plan for decode rows (up to 8 rows, or 16
    # with more than 8 chunks): the same fp32 chains
    for M, K in ((6, 4096), (16, 2048), (5, 640), (3, 8192)):
        G, N = 2, 128
        x, q, _ = _inputs(9400 + M, M, G, N, K)
        e32 = S.exponent_bytes(S.rng(9401 + M), (G, N // 32, K // 32), 112, 128)
        e_rows = np.repeat(e32, 32, axis=1)
        y32 = bf16_bits(B.bsfp8_gemm(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e32)))
        yr = bf16_bits(B.bsfp8_gemm_row32(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e_rows)))
        assert np.array_equal(y32, yr), (M, K)


def test_integer_exact_inputs_bitwise_and_determinism():
    M, G, N, K = 12, 1, 64, 2048
    r = S.rng(9500)
    x = S.small_int_bf16(r, (M, G * K))
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], dtype=np.uint8)
    q = ints[r.integers(0, 8, (G, N, K))]
    e = np.full((G, N, K // 32), 127, dtype=np.uint8)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    y = B.bsfp8_gemm_row32(xt, qt, et, out_dtype="f32")
    assert np.array_equal(y.cpu().numpy(), R.gemm_row32(x, G, N, K, q, e, out="f32"))
    x, q, e = _inputs(9501, 16, 1, 1280, 5120)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    ws = B.workspace_row32(16, 1, 1280, 5120)
    ref = bf16_bits(B.bsfp8_gemm_row32(xt, qt, et, ws=ws))
    for _ in range(30):
        assert np.array_equal(bf16_bits(B.bsfp8_gemm_row32(xt, qt, et, ws=ws)), ref)


def test_row32_errors():
    x = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 64, 256), dtype=torch.uint8, device="cuda")
    e = torch.zeros((1, 64, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.BsfpError) as ei:                 # more than 16 rows
        B.bsfp8_gemm_row32(x, q, e)
    assert ei.value.status == B.ESHAPE
    with pytest.raises(B.BsfpError) as ei:                 # K not a multiple of 128
        B.bsfp8_gemm_row32(x[:4, :160].contiguous(), q[:, :, :160].contiguous(), e[:, :, :5].contiguous())
    assert ei.value.status == B.ESHAPE
    with pytest.raises(B.BsfpError) as ei:                 # a 32x32 configuration on the row-scale entry
        B.bsfp8_gemm_row32_config(x[:4], q, e, 54, 2)
    assert ei.value.status == B.EINVAL
