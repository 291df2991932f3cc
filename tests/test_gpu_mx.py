"""GPU parity of the MXFP8 path (activation quantizer and fp8 x fp8 GEMM) against the CPU oracle
(oracle/mx.py), through the C ABI. Codes and scale bytes must match bit for bit; GEMM outputs
follow the rule of parity.check_mx_bf16 / check_mx_f32 (the block-scaled fp8 MFMA is not an exact
sum rounded once), with integer-exact and one-hot inputs bitwise."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import oracle.mx as MX
import synthetic as S
from parity import bf16_bits, check_mx_bf16, check_mx_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _quant_gpu(x_bits, L=None):
    xq, xs = B.bsfp8_quantize_mx(to_gpu_bf16(x_bits), L)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def test_quantize_random_rows_bitwise():
    r = S.rng(8100)
    for M, L, scale in ((1, 32, 1.0), (7, 8192, 1.0), (33, 5120, 1e-3), (5, 640, 3e4)):
        x = S.bf16_normal(r, (M, L), scale=scale)
        q, s = _quant_gpu(x)
        rq, rs = MX.quantize_mx(x)
        assert np.array_equal(q, rq) and np.array_equal(s, rs), (M, L)


def test_quantize_strided_rows_and_a_prefix():
    x = S.bf16_normal(S.rng(8101), (9, 1024 + 96))
    q, s = _quant_gpu(x[:, :1024].copy())
    xt = to_gpu_bf16(x)
    q2, s2 = B.bsfp8_quantize_mx(xt, 1024)
    rq, rs = MX.quantize_mx(x, 1024)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    assert np.array_equal(q2.cpu().numpy(), rq) and np.array_equal(s2.cpu().numpy(), rs)


def test_quantize_every_bf16_magnitude_and_edge_blocks():
    # every finite positive bf16 pattern once, in random sign and order, 32 per block: covers the
    # scale rule at every exponent, subnormal amax, saturation and ties
    mags = np.arange(1, 0x7F80, dtype=np.uint16)
    r = S.rng(8102)
    vals = r.permutation(mags)
    n = (len(vals) // 1024) * 1024
    x = (vals[:n] | (r.integers(0, 2, n).astype(np.uint16) << 15)).reshape(-1, 1024)
    x = np.concatenate([x, np.pad(vals[n:], (0, 1024 - (len(vals) - n)))[None, :]])
    q, s = _quant_gpu(x)
    rq, rs = MX.quantize_mx(x)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    # blocks of one magnitude pattern each (amax = that pattern): every scale exponent
    one = np.repeat(np.arange(0, 0x7F80, 7, dtype=np.uint16)[:, None], 32, axis=1)
    one[:, 1::2] |= 0x8000
    q, s = _quant_gpu(one)
    rq, rs = MX.quantize_mx(one)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    # zero, signed-zero, subnormal-only, saturating and non-finite blocks
    edge = np.zeros((6, 32), dtype=np.uint16)
    edge[1, ::2] = 0x8000
    edge[2, :] = np.arange(1, 33, dtype=np.uint16)              # bf16 subnormals
    edge[3, :] = oracle.f64_to_bf16_bits(np.linspace(-511.0, 511.0, 32) * 2.0 ** -8 * 2.0 ** 8)
    edge[4, 5] = 0x7F80                                          # +inf in a block
    edge[5, 9] = 0xFFC1                                          # NaN in a block
    edge[4, 6] = 0xBF80
    q, s = _quant_gpu(edge)
    rq, rs = MX.quantize_mx(edge)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    assert s[4, 0] == 255 and s[5, 0] == 255 and q[4, 6] == 0xFF


def _mx_inputs(seed, M, G, N, K, elo=115, ehi=125, xscale=1.0):
    r = S.rng(seed)
    x = S.bf16_normal(r, (M, G * K), scale=xscale)
    xq, xs = MX.quantize_mx(x)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), elo, ehi)
    return xq, xs, q, e


def _gemm_mx(xq, xs, q, e, cfg=None, out_dtype="bf16"):
    args = (to_gpu_u8(xq), to_gpu_u8(xs), to_gpu_u8(q), to_gpu_u8(e))
    y = B.bsfp8_gemm_mx(*args, out_dtype=out_dtype) if cfg is None else \
        B.bsfp8_gemm_mx_config(*args, cfg, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,G,N,K", [(1, 1, 32, 128), (6, 2, 1024, 4096), (16, 1, 64, 640), (40, 2, 128, 1024),
                                     (100, 1, 96, 512), (192, 1, 64, 1152), (256, 1, 32, 256),
                                     (24, 1, 2048, 5120)])
def test_gemm_mx_parity(M, G, N, K):
    xq, xs, q, e = _mx_inputs(8200 + M + K, M, G, N, K)
    exact = MX.gemm_mx_exact_f64(xq, xs, G, N, K, q, e)
    absum = MX.abs_products_sum_mx(xq, xs, G, N, K, q, e)
    y = _gemm_mx(xq, xs, q, e)
    assert y.shape == (M, G, N)
    st = check_mx_bf16(bf16_bits(y), exact, absum, K)
    print(f"M={M} G={G} N={N} K={K} cfg {B.bsfp8_mx_plan(M, G, N)}: {st}")


@pytest.mark.parametrize("N,K", [(256, 640), (256, 1024), (128, 8192)])
def test_every_mx_configuration(N, K):
    """Each compiled configuration on a shape with several m-blocks, a ragged last m-block and a
    partial last ring stage, bf16 and fp32 outputs; K with an odd (5), an even (8) and the
    largest (64) chunk count, which decide the row stride of the staged activation scales."""
    G = 2
    for cfg in range(B.bsfp8_mx_num_configs()):
        info = B.bsfp8_mx_config_info(cfg)
        M = min(2 * info["BM"] - 3, 256)
        xq, xs, q, e = _mx_inputs(8300 + cfg + K, M, G, N, K)
        exact = MX.gemm_mx_exact_f64(xq, xs, G, N, K, q, e)
        absum = MX.abs_products_sum_mx(xq, xs, G, N, K, q, e)
        print(f"mx cfg {cfg} {info} M {M} N {N} K {K}", flush=True)
        check_mx_bf16(bf16_bits(_gemm_mx(xq, xs, q, e, cfg)), exact, absum, K)
        rel = check_mx_f32(_gemm_mx(xq, xs, q, e, cfg, "f32").cpu().numpy(), exact, absum, K)
        print(f"    fp32 max |err|/sum|xw| = {rel:.3e} (2^{np.log2(max(rel, 1e-300)):.1f})")


def test_integer_exact_and_one_hot_inputs_are_bitwise():
    # small integers with unit scales: every partial sum is an exact small integer, inside the
    # MFMA's window, so the fp32 result is exact and its bf16 rounding equals the oracle's
    M, G, N, K = 20, 2, 96, 1024
    r = S.rng(8400)
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], dtype=np.uint8)   # 0, 1, 2, 3, 4, -1, -2, -3
    xq = ints[r.integers(0, 8, (M, G * K))]
    xs = np.full((M, G * K // 32), 127, dtype=np.uint8)
    q = ints[r.integers(0, 8, (G, N, K))]
    e = np.full((G, N // 32, K // 32), 127, dtype=np.uint8)
    y = _gemm_mx(xq, xs, q, e, out_dtype="f32").cpu().numpy()
    assert np.array_equal(y, MX.gemm_mx(xq, xs, G, N, K, q, e, out="f32"))
    # one-hot rows (a single 1.0 code, scale byte 127) give the weights themselves, bitwise
    xq = np.zeros((M, G * K), dtype=np.uint8)
    for m in range(M):
        xq[m, (m * 97) % (G * K)] = 0x38
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 115, 125)
    y = bf16_bits(_gemm_mx(xq, xs, q, e))
    # compared as values: the sign of an exactly-zero sum is not fixed by the pages
    assert np.array_equal(oracle.bf16_bits_to_f64(y), oracle.bf16_bits_to_f64(MX.gemm_mx(xq, xs, G, N, K, q, e)))


def test_quantize_then_gemm_end_to_end_and_determinism():
    M, G, N, K = 6, 2, 1024, 4096
    d = S.wo_a(8500, M, G, N, K)
    xt = to_gpu_bf16(d["x"])
    xq, xs = B.bsfp8_quantize_mx(xt)
    rq, rs = MX.quantize_mx(d["x"])
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    qg, eg = to_gpu_u8(d["q"]), to_gpu_u8(d["e"])
    y0 = B.bsfp8_gemm_mx(xq, xs, qg, eg)
    exact = MX.gemm_mx_exact_f64(rq, rs, G, N, K, d["q"], d["e"])
    absum = MX.abs_products_sum_mx(rq, rs, G, N, K, d["q"], d["e"])
    check_mx_bf16(bf16_bits(y0), exact, absum, K)
    ref = bf16_bits(y0)
    for _ in range(20):
        assert np.array_equal(bf16_bits(B.bsfp8_gemm_mx(xq, xs, qg, eg)), ref)


def test_mx_errors_and_empty():
    xq = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((4, 8), dtype=torch.uint8, device="cuda")
    q = torch.zeros((1, 64, 256), dtype=torch.uint8, device="cuda")
    e = torch.zeros((1, 2, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.BsfpError) as ei:           # K not a multiple of 128
        B.bsfp8_gemm_mx(xq[:, :160], xs[:, :5], q[:, :, :160].contiguous(), e[:, :, :5].contiguous())
    assert ei.value.status in (B.ESHAPE, B.ESTRIDE)
    y = B.bsfp8_gemm_mx(xq[:0], xs[:0], q, e)
    assert y.shape == (0, 1, 64)
