"""GPU parity of the MXFP8 output epilogue (oracle/epilogue.py) through the C ABI:
  * the fused sum-and-quantise kernel on seeded fp32 partials, both orders, 1..64 partials, with
    zero, non-finite, saturating, tie and far-out-of-range blocks: bit for bit;
  * the GEMM with the epilogue on integer-exact inputs (every fp32 sum exact): bit for bit, for
    every kernel kind and with split partials;
  * on random inputs at the workloads' sizes: the rule of parity.check_mxfp8 against the ideal
    epilogue of the exact product, and bitwise agreement with quantising bsfp8_gemm's own fp32
    output (the epilogue sums the partials in the plan's own order);
  * HIP-graph replay equal to the eager result."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import oracle.epilogue as EP
import synthetic as S
from parity import check_mxfp8, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu

ORDERS = (B.SUM_ASCENDING, B.SUM_PAIRWISE)


def _partials(seed, S_, M, L):
    """fp32 partials [S, M, L]: normals times a power of two per (partial, row, block) over a wide
    range, plus blocks that exercise the quantiser's edges."""
    r = S.rng(seed)
    p = S.f32_normal(r, (S_, M, L))
    sc = np.ldexp(np.float32(1.0), r.integers(-140, 100, size=(S_, M, L // 32))).astype(np.float32)
    p = (p * np.repeat(sc, 32, axis=2)).astype(np.float32)
    nb = M * (L // 32)
    blocks = p.reshape(S_, nb, 32)
    if nb >= 8:
        blocks[:, 0] = 0.0                                          # all-zero block
        blocks[:, 1, 3] = np.float32(-0.0)
        blocks[0, 2, 7] = np.nan                                    # non-finite blocks
        blocks[S_ - 1, 3, 0] = -np.inf
        blocks[:, 4] = 0.0                                          # a tie after scaling (1.0625)
        blocks[0, 4, 0], blocks[0, 4, 1] = 1.0, np.float32(1.0625 / 256)
        blocks[:, 5] = 0.0                                          # saturation: 1.9 * 2^8 > 448
        blocks[0, 5, 0], blocks[0, 5, 1] = np.float32(1.9), np.float32(-1.9)
        with np.errstate(over="ignore"):                            # near and past the top of
            blocks[:, 6] *= np.float32(2.0 ** 100)                  # fp32 (some become inf)
        blocks[:, 7] = np.ldexp(np.float32(1), -149) * r.integers(-3, 4, size=(S_, 32))   # subnormals
    return blocks.reshape(S_, M, L)


@pytest.mark.parametrize("S_", [1, 2, 3, 5, 8, 13, 64])
@pytest.mark.parametrize("order", ORDERS)
def test_reduce_quantize_bitwise(S_, order):
    for M, L in ((1, 32), (3, 96), (7, 2048)):
        if S_ == 64 and M * L > 4096:
            continue
        part = _partials(9000 + 31 * S_ + M, S_, M, L)
        print(f"reduce_quantize S={S_} order={order} M={M} L={L}", flush=True)
        yq, ys = B.bsfp8_reduce_quantize_mx(torch.from_numpy(part).cuda(), order)
        torch.cuda.synchronize()
        rq, rs = EP.reduce_quantize_mx(part, order)
        assert np.array_equal(ys.cpu().numpy(), rs), (S_, order, M, L)
        assert np.array_equal(yq.cpu().numpy(), rq), (S_, order, M, L)


def test_reduce_quantize_every_fp32_binade():
    # one block per fp32 exponent field (random mantissas and signs): every scale exponent,
    # subnormal maxima and the clamp at -127
    r = S.rng(9050)
    E = np.arange(0, 255, dtype=np.uint32)
    mant = r.integers(0, 1 << 23, size=(E.size, 32)).astype(np.uint32)
    sign = r.integers(0, 2, size=(E.size, 32)).astype(np.uint32) << 31
    bits = sign | (E[:, None] << 23) | mant
    bits[:, 1:] = (bits[:, 1:] & 0x80000000) | ((bits[:, 1:] & 0x7FFFFFFF) >> r.integers(0, 12, size=(E.size, 31)).astype(np.uint32))
    part = bits.view(np.float32)[None]
    yq, ys = B.bsfp8_reduce_quantize_mx(torch.from_numpy(np.ascontiguousarray(part)).cuda(), B.SUM_ASCENDING)
    torch.cuda.synchronize()
    rq, rs = EP.reduce_quantize_mx(part, B.SUM_ASCENDING)
    assert np.array_equal(ys.cpu().numpy(), rs) and np.array_equal(yq.cpu().numpy(), rq)


def _int_case(seed, M, G, N, K):
    """Small-integer activations and integer-valued weight codes at unit scale: every partial and
    every sum is an integer below 2^24, exact in fp32 in any order."""
    r = S.rng(seed)
    x = S.small_int_bf16(r, (M, G * K), -2, 2)
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], dtype=np.uint8)   # 0..8
    q = ints[r.integers(0, ints.size, size=(G, N, K))] | (r.integers(0, 2, size=(G, N, K)).astype(np.uint8) << 7)
    e = np.full((G, N // 32, K // 32), 127, dtype=np.uint8)
    return x, q, e


# (M, G, N, K, split_k): the decode kernel (with and without split partials), the direct kernel
# (ragged K), the slab and rows kernels, and the tile kernel with split partials (ascending order)
INT_CASES = [(6, 2, 1024, 4096, 0), (6, 2, 1024, 4096, 2), (8, 2, 1024, 4096, 5), (3, 1, 5120, 576, 0),
             (13, 1, 1024, 2048, 0), (48, 2, 1024, 4096, 0), (130, 2, 1024, 4096, 0),
             (16, 1, 16384, 1024, 0), (16, 1, 16384, 1024, 3)]


@pytest.mark.parametrize("M,G,N,K,sk", INT_CASES)
def test_gemm_mxfp8_integer_exact_bitwise(M, G, N, K, sk):
    x, q, e = _int_case(9100 + M + sk, M, G, N, K)
    plan = B.bsfp8_plan_info(M, G, N, K, split_k=sk, path=3)
    print(f"gemm_mxfp8 int M={M} G={G} N={N} K={K} split={sk} plan {plan}", flush=True)
    yq, ys = B.bsfp8_gemm_mxfp8(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e), split_k=sk)
    torch.cuda.synchronize()
    rq, rs, Y = EP.gemm_mxfp8_ideal(x, G, N, K, q, e)
    assert np.array_equal(Y, np.round(Y)) and np.abs(Y).max() < 2 ** 24
    assert np.array_equal(ys.cpu().numpy(), rs)
    assert np.array_equal(yq.cpu().numpy(), rq)


@pytest.fixture(scope="module")
def wo_a_weight():
    d = S.wo_a(2000, 1)
    W = oracle.dequant_values(d["q"], d["e"])
    return d, W, np.abs(W), to_gpu_u8(d["q"]), to_gpu_u8(d["e"])


def _exact_and_absum(x, W, Wabs, G, K):
    M = x.shape[0]
    X = oracle.bf16_bits_to_f64(x[:, : G * K]).reshape(M, G, K)
    Y = np.stack([X[:, g] @ W[g].T for g in range(G)], axis=1)
    A = np.stack([np.abs(X[:, g]) @ Wabs[g].T for g in range(G)], axis=1)
    return Y.reshape(M, -1), A.reshape(M, -1)


@pytest.mark.parametrize("M,sk", [(1, 0), (2, 0), (6, 0), (6, 2), (6, 4), (8, 0), (16, 0), (64, 0), (192, 0)])
def test_gemm_mxfp8_wo_a_full_size(wo_a_weight, M, sk):
    d, W, Wabs, qt, et = wo_a_weight
    G, N, K = 2, 1024, 4096
    x = S.bf16_normal(S.rng(9200 + M), (M, G * K))
    plan = B.bsfp8_plan_info(M, G, N, K, split_k=sk, path=3)
    print(f"gemm_mxfp8 wo_a M={M} split={sk} plan {plan}", flush=True)
    xt = to_gpu_bf16(x)
    yq, ys = B.bsfp8_gemm_mxfp8(xt, qt, et, split_k=sk)
    # the same plan's fp32 output, quantised by the stand-alone epilogue with one partial
    y32 = B.bsfp8_gemm_config(xt, qt, et, plan["cfg"], plan["cps"], out_dtype="f32")
    q2, s2 = B.bsfp8_reduce_quantize_mx(y32.reshape(1, M, G * N), B.SUM_ASCENDING)
    torch.cuda.synchronize()
    assert torch.equal(yq, q2) and torch.equal(ys, s2)
    Y, A = _exact_and_absum(x, W, Wabs, G, K)
    stats = check_mxfp8(yq.cpu().numpy(), ys.cpu().numpy(), Y, A, K, plan["splits"])
    print(stats, flush=True)
    assert stats["same"] >= stats["n"] * 0.99


def test_gemm_mxfp8_shared_down_and_lm_head_rows():
    # ragged K (the direct kernel) and the wide LM-head shape (the tile kernel), sampled rows
    d = S.shared_down(9300, M=6)
    e = oracle.scales_from_f32(d["scales"])[None]
    W = oracle.dequant_values(d["q"], e)
    yq, ys = B.bsfp8_gemm_mxfp8(to_gpu_bf16(d["x"]), to_gpu_u8(d["q"]), to_gpu_u8(e))
    torch.cuda.synchronize()
    Y, A = _exact_and_absum(d["x"], W, np.abs(W), 1, 576)
    print(check_mxfp8(yq.cpu().numpy(), ys.cpu().numpy(), Y, A, 576), flush=True)
    h = S.lm_head(9301, 16, N=16384)
    yq, ys = B.bsfp8_gemm_mxfp8(to_gpu_bf16(h["x"]), to_gpu_u8(h["q"]), to_gpu_u8(h["e"]), split_k=2)
    torch.cuda.synchronize()
    rows = [0, 7, 15]
    W = oracle.dequant_values(h["q"], h["e"])
    Y, A = _exact_and_absum(h["x"][rows], W, np.abs(W), 1, 5120)
    print(check_mxfp8(yq.cpu().numpy()[rows], ys.cpu().numpy()[rows], Y, A, 5120), flush=True)


# decode shapes where the built-in plan is the 16-row decode kernel with one split: the fused
# kernel runs (32 weight rows per workgroup, GEMM and epilogue in one launch); the explicit
# configuration call takes the two-kernel form with the same plan, so both must agree bitwise
FUSED_CASES = [(1, 2, 1024, 4096), (6, 2, 1024, 4096), (8, 2, 1024, 4096), (13, 2, 1024, 4096),
               (16, 2, 1024, 4096), (6, 4, 1024, 4096), (6, 1, 5120, 640), (5, 1, 96, 384), (3, 1, 64, 1152),
               (9, 1, 32, 1280), (4, 1, 32, 128), (1, 3, 96, 256), (2, 1, 64, 4096)]


@pytest.mark.parametrize("M,G,N,K", FUSED_CASES)
def test_fused_decode_equals_the_two_kernel_form(M, G, N, K):
    r = S.rng(9500 + M + K)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 112, 126)
    plan = B.bsfp8_plan_info(M, G, N, K, path=3)
    info = B.bsfp8_config_info(plan["cfg"])
    print(f"fused M={M} G={G} N={N} K={K} plan {plan} kind {info['kind']}", flush=True)
    assert info["kind"] == 4 and plan["splits"] == 1
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    yq, ys = B.bsfp8_gemm_mxfp8(xt, qt, et)
    q2, s2 = B.bsfp8_gemm_mxfp8_config(xt, qt, et, plan["cfg"], plan["cps"])
    torch.cuda.synchronize()
    assert torch.equal(ys, s2) and torch.equal(yq, q2)
    W = oracle.dequant_values(q, e)
    Y, A = _exact_and_absum(x, W, np.abs(W), G, K)
    print(check_mxfp8(yq.cpu().numpy(), ys.cpu().numpy(), Y, A, K, 1), flush=True)


# plans whose own kernel quantises its output (one split, 32-column blocks per wave or per
# workgroup): the LDS-staged register kernel (33..192 rows, K of at most 32 whole chunks), the
# slab kernel (33..64 rows, longer K), the rows kernel (ragged K, or more than 192 rows) and the
# tile kernel (wide weights); the explicit configuration call takes the two-kernel form of the
# same plan
IN_KERNEL_CASES = [(33, 2, 1024, 4096, 8), (64, 1, 256, 2048, 8), (65, 2, 1024, 4096, 8), (128, 1, 512, 1024, 8),
                   (160, 1, 256, 2048, 8), (33, 1, 256, 5120, 5), (64, 1, 256, 8192, 5), (65, 2, 1024, 4000, 2),
                   (128, 1, 512, 1056, 2), (200, 1, 256, 1152, 2), (256, 1, 64, 256, 2), (16, 1, 16384, 1024, 3),
                   (64, 1, 16384, 512, 3), (100, 1, 16384, 256, 3)]


@pytest.mark.parametrize("M,G,N,K,kind", IN_KERNEL_CASES)
def test_in_kernel_epilogue_equals_the_two_kernel_form(M, G, N, K, kind):
    r = S.rng(9600 + M + N)
    x = S.bf16_normal(r, (M, G * K))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 112, 126)
    plan = B.bsfp8_plan_info(M, G, N, K, path=3)
    info = B.bsfp8_config_info(plan["cfg"])
    print(f"in-kernel M={M} G={G} N={N} K={K} plan {plan} kind {info['kind']}", flush=True)
    assert info["kind"] == kind and plan["splits"] == 1
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    yq, ys = B.bsfp8_gemm_mxfp8(xt, qt, et)
    q2, s2 = B.bsfp8_gemm_mxfp8_config(xt, qt, et, plan["cfg"], plan["cps"])
    torch.cuda.synchronize()
    assert torch.equal(ys, s2) and torch.equal(yq, q2)
    rows = list(range(0, M, max(1, M // 7)))[:8]
    W = oracle.dequant_values(q, e)
    Y, A = _exact_and_absum(x[rows], W, np.abs(W), G, K)
    print(check_mxfp8(yq.cpu().numpy()[rows], ys.cpu().numpy()[rows], Y, A, K, 1), flush=True)


def test_gemm_mxfp8_graph_replay_and_repeats(wo_a_weight):
    d, W, Wabs, qt, et = wo_a_weight
    M, G, N, K = 6, 2, 1024, 4096
    xt = to_gpu_bf16(S.bf16_normal(S.rng(9400), (M, G * K)))
    ws = B.workspace_mxfp8(M, G, N, K)
    yq0, ys0 = B.bsfp8_gemm_mxfp8(xt, qt, et, ws=ws)
    yq0, ys0 = yq0.clone(), ys0.clone()
    for _ in range(20):
        yq, ys = B.bsfp8_gemm_mxfp8(xt, qt, et, ws=ws)
        assert torch.equal(yq, yq0) and torch.equal(ys, ys0)
    yq, ys = torch.empty_like(yq0), torch.empty_like(ys0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.bsfp8_gemm_mxfp8(xt, qt, et, ws=ws, yq=yq, ys=ys)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.bsfp8_gemm_mxfp8(xt, qt, et, ws=ws, yq=yq, ys=ys)
    for _ in range(3):
        yq.zero_()
        ys.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yq, yq0) and torch.equal(ys, ys0)


def test_gemm_mxfp8_empty_and_errors():
    G, N, K = 1, 64, 128
    q = torch.zeros((G, N, K), dtype=torch.uint8, device="cuda")
    e = torch.full((G, N // 32, K // 32), 127, dtype=torch.uint8, device="cuda")
    yq, ys = B.bsfp8_gemm_mxfp8(torch.zeros((0, K), dtype=torch.bfloat16, device="cuda"), q, e)
    assert yq.shape == (0, G * N) and ys.shape == (0, G * N // 32)
    x = torch.zeros((4, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):                          # workspace too small (binding)
        B.bsfp8_gemm_mxfp8(x, q, e, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    n = B.bsfp8_workspace_bytes_mxfp8(4, G, N, K)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    yq4 = torch.empty((4, G * N), dtype=torch.uint8, device="cuda")
    ys4 = torch.empty((4, G * N // 32), dtype=torch.uint8, device="cuda")
    st = B.lib().bsfp8_gemm_mxfp8(B._ptr(x), K, 4, G, N, K, B._ptr(q), B._ptr(e), 0, B._ptr(ws), n - 16,
                                  B._ptr(yq4), B._ptr(ys4), B._stream(x))   # ... and the library
    assert st == B.EWORKSPACE
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_gemm_mxfp8(torch.zeros((257, K), dtype=torch.bfloat16, device="cuda"), q, e)
    assert ei.value.status == B.ESHAPE
    part = torch.zeros((65, 1, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_reduce_quantize_mx(part)
    assert ei.value.status == B.EINVAL
    # an all-zero product: scale byte 0 and zero codes
    yq, ys = B.bsfp8_gemm_mxfp8(x, q, e)
    torch.cuda.synchronize()
    assert int(yq.abs().sum()) == 0 and int(ys.sum()) == 0
