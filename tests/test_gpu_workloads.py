"""GPU parity at the workloads' full sizes, through the C ABI, with the built-in plans that the
benchmark times: the shared-expert down_proj (K 576 and padded 640), the wo_a decode and mid
shapes at G=2, a padded-TP3 wo_a layer built by the twin encoder (clean and perturbed) then used
at G=4, and the draft LM head's fp32 logits on sampled output rows with per-row batch
invariance."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import synthetic as S
from parity import bf16_bits, check_bf16, check_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _exact(x, W, G, K):
    """float64 Y from X bits and dequantised weights W [G, N, K] (float64 values)."""
    M = x.shape[0]
    X = oracle.bf16_bits_to_f64(x[:, : G * K]).reshape(M, G, K)
    return np.stack([X[:, g] @ W[g].T for g in range(G)], axis=1)


@pytest.fixture(scope="module")
def wo_a_weight():
    d = S.wo_a(2000, 1)
    W = oracle.dequant_values(d["q"], d["e"])
    return d, W, to_gpu_u8(d["q"]), to_gpu_u8(d["e"])


@pytest.mark.parametrize("M", [2, 4, 6, 8, 16, 24, 32, 64, 128, 192])
def test_wo_a_full_size(wo_a_weight, M):
    d, W, qt, et = wo_a_weight
    x = S.bf16_normal(S.rng(2100 + M), (M, 2 * 4096))
    print(f"wo_a M={M} plan {B.bsfp8_plan_info(M, 2, 1024, 4096)}", flush=True)
    y = B.bsfp8_gemm(to_gpu_bf16(x), qt, et)
    torch.cuda.synchronize()
    stats = check_bf16(bf16_bits(y), x, 2, 1024, 4096, d["q"], d["e"], exact=_exact(x, W, 2, 4096))
    assert stats["within_1ulp"] >= stats["n"] - 50


def test_shared_down_full_size_and_padding():
    d = S.shared_down(1000, M=6)
    e = oracle.scales_from_f32(d["scales"], 5120, 576)[None]
    eg = B.bsfp8_scales_from_f32(torch.from_numpy(d["scales"]).cuda())[None]
    assert np.array_equal(eg.cpu().numpy(), e)
    q = to_gpu_u8(d["q"])
    x = to_gpu_bf16(d["x"])
    y = B.bsfp8_gemm(x, q, eg)
    qp, ep = B.bsfp8_pad_k_weight(q, eg, 640)
    y640 = B.bsfp8_gemm(B.bsfp8_pad_k_input(x, 1, 576, 640), qp, ep)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y640.view(torch.int16))
    check_bf16(bf16_bits(y), d["x"], 1, 5120, 576, d["q"], e)


def test_twin_layer_tp3_then_gemm():
    src = S.twin_source(4000, G=4, R=1024, D=4096)
    w = oracle.dequant_bf16(src["q"], src["e"])
    wt = to_gpu_bf16(w)
    t = B.bsfp8_make_twin(wt)
    ref = oracle.make_twin(w)
    assert t.accepted and ref.accepted
    assert np.array_equal(t.q.cpu().numpy(), ref.q) and np.array_equal(t.e.cpu().numpy(), ref.e)
    # the same layer with 10% of its blocks perturbed by one bf16 ulp: rejected block by block
    wp, mask = S.perturb_one_element(w, S.rng(4001), 0.1)
    tp = B.bsfp8_make_twin(to_gpu_bf16(wp))
    refp = oracle.make_twin(wp)
    assert not tp.accepted and not refp.accepted
    assert np.array_equal(tp.ok.cpu().numpy(), refp.ok) and np.array_equal(refp.ok.astype(bool), ~mask)
    assert np.array_equal(tp.e.cpu().numpy(), refp.e) and np.array_equal(tp.q.cpu().numpy(), refp.q)
    assert tp.n_bad == int(mask.sum())
    # the accepted twin feeds the GEMM at G = 4
    W = oracle.dequant_values(ref.q, ref.e)
    for M in (2, 6, 8):
        x = S.bf16_normal(S.rng(4100 + M), (M, 4 * 4096))
        y = B.bsfp8_gemm(to_gpu_bf16(x), t.q, t.e)
        torch.cuda.synchronize()
        check_bf16(bf16_bits(y), x, 4, 1024, 4096, ref.q, ref.e, exact=_exact(x, W, 4, 4096))


def test_lm_head_sampled_rows_and_batch_invariance():
    N, K = 32768, 5120
    d = S.lm_head(5000, 128)
    qt, et = to_gpu_u8(d["q"]), to_gpu_u8(d["e"])
    xt = to_gpu_bf16(d["x"])
    ys = {}
    for M in (16, 64, 128):
        print(f"lm_head M={M} plan {B.bsfp8_plan_info(M, 1, N, K)}", flush=True)
        ys[M] = B.bsfp8_gemm(xt[:M], qt, et, out_dtype="f32")
    torch.cuda.synchronize()
    # the same row gives the same fp32 logits whatever the batch
    assert torch.equal(ys[16], ys[64][:16]) and torch.equal(ys[64], ys[128][:64])
    # sampled 32-row blocks of the vocabulary, checked against the oracle
    blocks = [0, 1, 333, 512, 777, 1023]
    rows = np.concatenate([np.arange(b * 32, b * 32 + 32) for b in blocks])
    q_s = d["q"][:, rows]
    e_s = d["e"][:, blocks]
    y128 = ys[128].cpu().numpy()[:, :, rows]
    check_f32(y128, d["x"], 1, rows.size, K, q_s, e_s)
    # and the bf16 rounding of those logits under the bf16 rule
    check_bf16(oracle.f64_to_bf16_bits(y128.astype(np.float64)), d["x"], 1, rows.size, K, q_s, e_s)


# ---- the fp8 x fp8 path and the row-scale twin at their full sizes -------------------------------
def test_mx_path_full_sizes_and_graph_replay():
    """The fp8 x fp8 path at the wo_a mid shape (M = 192, every output) and the LM head (M = 128,
    sampled vocabulary blocks), in the plans the benchmark times, plus a captured graph of
    quantizer + GEMM replayed against the eager result."""
    import oracle.mx as MX
    from parity import check_mx_bf16, check_mx_f32
    # wo_a mid, 192 rows: quantizer bitwise, every output under the fp8 rule
    d = S.wo_a(8600, 192)
    xt = to_gpu_bf16(d["x"])
    xq, xs = B.bsfp8_quantize_mx(xt)
    rq, rs = MX.quantize_mx(d["x"])
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    qt, et = to_gpu_u8(d["q"]), to_gpu_u8(d["e"])
    y = B.bsfp8_gemm_mx(xq, xs, qt, et)
    exact = MX.gemm_mx_exact_f64(rq, rs, 2, 1024, 4096, d["q"], d["e"])
    absum = MX.abs_products_sum_mx(rq, rs, 2, 1024, 4096, d["q"], d["e"])
    print("mx wo_a_mid M=192", check_mx_bf16(bf16_bits(y), exact, absum, 4096), flush=True)
    # graph replays of quantize + GEMM equal the eager result
    out = torch.empty_like(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.bsfp8_quantize_mx(xt, xq=xq, xs=xs)
        B.bsfp8_gemm_mx(xq, xs, qt, et, out=out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.bsfp8_quantize_mx(xt, xq=xq, xs=xs)
        B.bsfp8_gemm_mx(xq, xs, qt, et, out=out)
    for i in range(4):
        out.fill_(0)
        xq.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y.view(torch.int16)), i
        B.bsfp8_gemm_mx(xq, xs, qt, et)                  # eager work between replays
        torch.cuda.synchronize()
    # LM head, 128 rows, fp32 logits on sampled 32-row vocabulary blocks
    N, K = 32768, 5120
    d = S.lm_head(8700, 128)
    xq, xs = B.bsfp8_quantize_mx(to_gpu_bf16(d["x"]))
    rq, rs = MX.quantize_mx(d["x"])
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    y = B.bsfp8_gemm_mx(xq, xs, to_gpu_u8(d["q"]), to_gpu_u8(d["e"]), out_dtype="f32").cpu().numpy()
    blocks = [0, 5, 400, 1023]
    rows = np.concatenate([np.arange(b * 32, b * 32 + 32) for b in blocks])
    q_s, e_s = d["q"][:, rows], d["e"][:, blocks]
    exact = MX.gemm_mx_exact_f64(rq, rs, 1, rows.size, K, q_s, e_s)
    absum = MX.abs_products_sum_mx(rq, rs, 1, rows.size, K, q_s, e_s)
    rel = check_mx_f32(y[:, :, rows], exact, absum, K)
    print(f"mx lm_head M=128 sampled: max |err|/sum|xw| = {rel:.3e}", flush=True)


@pytest.mark.parametrize("M", [1, 6, 16])
def test_row32_main_proj_full_size(M):
    """The row-scale twin at the draft main_proj shard: a 1280 x 5120 weight built exact, encoded
    by the GPU encoder (bitwise vs the oracle), then the GEMV at 1, 6 and 16 rows."""
    import oracle.row32 as R
    from parity import check_bf16_exact
    r = S.rng(8800)
    q = S.e4m3_codes(r, (1, 1280, 5120))
    e = S.exponent_bytes(r, (1, 1280, 160), 115, 125)
    w = R.dequant_bf16_row32(q, e)
    t = B.bsfp8_make_twin_row32(to_gpu_bf16(w))
    ref = R.make_twin_row32(w)
    assert t.accepted and ref.accepted
    assert np.array_equal(t.q.cpu().numpy(), ref.q) and np.array_equal(t.e.cpu().numpy(), ref.e)
    x = S.bf16_normal(S.rng(8801 + M), (M, 5120))
    y = B.bsfp8_gemm_row32(to_gpu_bf16(x), t.q, t.e)
    exact = R.gemm_exact_f64_row32(x, 1, 1280, 5120, ref.q, ref.e)
    st = check_bf16_exact(bf16_bits(y), exact, lambda: R.abs_products_sum_row32(x, 1, 1280, 5120, ref.q, ref.e), 5120)
    print(f"main_proj M={M}: {st}", flush=True)
