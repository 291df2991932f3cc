"""GPU parity of the preparation steps (scale ingestion, twin encoder, K padding, dequant)
against the CPU oracle, through the C ABI. Integer and byte outputs must match bit for bit."""
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import synthetic as S
from parity import bf16_bits, check_bf16, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_scales_golden_and_random():
    with open(os.path.join(GOLDEN, "scales.txt")) as f:
        rows = [ln.split("#", 1)[0].split() for ln in f if ln.split("#", 1)[0].strip()]
    for hexbits, verdict, byte in rows:
        s = torch.from_numpy(np.array([[int(hexbits, 16)]], dtype=np.uint32).view(np.int32)).view(torch.float32).cuda()
        if verdict == "ok":
            assert int(B.bsfp8_scales_from_f32(s).item()) == int(byte), hexbits
        else:
            with pytest.raises(B.BsfpError) as ei:
                B.bsfp8_scales_from_f32(s)
            assert ei.value.status == B.ESCALE and ei.value.n_bad == 1
    sc = S.pow2_scales_f32(S.rng(10), (160, 18), -10, -4)
    got = B.bsfp8_scales_from_f32(torch.from_numpy(sc).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.scales_from_f32(sc, 5120, 576))
    bad = sc.copy()
    bad[3, 4] = 0.75
    bad[100, 0] = -1.0
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_scales_from_f32(torch.from_numpy(bad).cuda())
    assert ei.value.n_bad == 2


def _twin_gpu(w_bits):
    t = B.bsfp8_make_twin(to_gpu_bf16(w_bits))
    return t.accepted, t.q.cpu().numpy(), t.e.cpu().numpy(), t.ok.cpu().numpy(), t.n_bad


def test_make_twin_exact_weights_bitwise():
    src = S.twin_source(3000, G=2, R=256, D=512)
    w = oracle.dequant_bf16(src["q"], src["e"])
    acc, q, e, ok, nbad = _twin_gpu(w)
    ref = oracle.make_twin(w)
    assert acc and ref.accepted and nbad == 0
    assert np.array_equal(q, ref.q) and np.array_equal(e, ref.e) and np.array_equal(ok, ref.ok)


def test_make_twin_perturbed_and_random_weights_bitwise():
    src = S.twin_source(3001, G=1, R=128, D=1024)
    w = oracle.dequant_bf16(src["q"], src["e"])
    wp, mask = S.perturb_one_element(w, S.rng(3002), 0.1)
    wr = S.bf16_normal(S.rng(3003), (1, 64, 256))           # general bf16: mostly not exact
    for ww in (wp, wr):
        acc, q, e, ok, nbad = _twin_gpu(ww)
        ref = oracle.make_twin(ww)
        assert acc == ref.accepted and not acc
        assert nbad == int((ref.ok == 0).sum())
        assert np.array_equal(e, ref.e) and np.array_equal(ok, ref.ok)
        assert np.array_equal(q, ref.q)
    assert np.array_equal(_twin_gpu(wp)[3].astype(bool), ~mask)


def test_make_twin_async_equals_the_synchronous_call_and_replays_in_a_graph():
    """The asynchronous encoder writes the twin bytes, exponents and block mask of the
    synchronous call, adds its inexact-block count to the caller's device counter (so one counter
    gathers several layers), and replays in a graph with the counter cleared by a kernel."""
    src = S.twin_source(3010, G=2, R=256, D=512)
    w = oracle.dequant_bf16(src["q"], src["e"])
    wp, mask = S.perturb_one_element(w, S.rng(3011), 0.1)
    ref, refp = oracle.make_twin(w), oracle.make_twin(wp)
    wt, wpt = to_gpu_bf16(w), to_gpu_bf16(wp)
    n_bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    q, e, ok = B.bsfp8_make_twin_async(wt, n_bad)
    torch.cuda.synchronize()
    assert int(n_bad.item()) == 0
    assert np.array_equal(q.cpu().numpy(), ref.q) and np.array_equal(e.cpu().numpy(), ref.e)
    assert np.array_equal(ok.cpu().numpy(), ref.ok)
    qp, ep, okp = B.bsfp8_make_twin_async(wpt, n_bad)
    q2, e2, _ = B.bsfp8_make_twin_async(wpt, n_bad, ok=False)        # no mask; the count adds up
    torch.cuda.synchronize()
    nb = int((refp.ok == 0).sum())
    assert nb == int(mask.sum()) > 0 and int(n_bad.item()) == 2 * nb
    assert np.array_equal(qp.cpu().numpy(), refp.q) and np.array_equal(ep.cpu().numpy(), refp.e)
    assert np.array_equal(okp.cpu().numpy(), refp.ok)
    assert torch.equal(q2, qp) and torch.equal(e2, ep)
    # in a graph: two layers, one counter each, cleared inside the graph by a kernel
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    outs = [(torch.empty_like(q), torch.empty_like(e), torch.empty_like(ok)) for _ in range(2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            cnt.zero_()
            for i, ww in enumerate((wt, wpt)):
                B.bsfp8_make_twin_async(ww, cnt[i:i + 1], *outs[i])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            for t in o:
                t.fill_(0xAB)
        cnt.fill_(12345)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert cnt.tolist() == [0, nb], rep
        assert torch.equal(outs[0][0], q) and torch.equal(outs[0][1], e) and torch.equal(outs[0][2], ok)
        assert torch.equal(outs[1][0], qp) and torch.equal(outs[1][1], ep) and torch.equal(outs[1][2], okp)


def test_make_twin_edge_blocks():
    w = np.zeros((1, 64, 96), dtype=np.uint16)
    w[0, 0, 40] = 0x8000                  # block (0,1): only a negative zero
    w[0, 1, 70] = 0x0001                  # block (0,2): bf16 subnormals
    w[0, 2, 71] = 0x8003
    w[0, 33, 5] = 0x7F80                  # block (1,0): +inf
    w[0, 40, 50] = 0x7FC0                 # block (1,1): NaN
    w[0, 35, 65] = 0x43E0                 # block (1,2): 448
    w[0, 36, 66] = 0x3F81                 # ... and an 8-significant-bit value
    acc, q, e, ok, nbad = _twin_gpu(w)
    ref = oracle.make_twin(w)
    assert np.array_equal(e, ref.e) and np.array_equal(ok, ref.ok) and np.array_equal(q, ref.q)
    assert ok.tolist() == [[[1, 1, 1], [0, 0, 0]]] and nbad == 3 and not acc


def test_make_twin_all_bf16_magnitudes_one_per_block():
    # every positive finite bf16 pattern as the amax of its own block (plus a few smaller
    # companions): the exponent rule and the encoder over the whole bf16 range
    pats = np.arange(1, 0x7F80, 3, dtype=np.uint16)
    nb = pats.size
    w = np.zeros((1, 32, 32 * nb), dtype=np.uint16)
    w[0, 0, 32 * np.arange(nb)] = pats
    w[0, 5, 32 * np.arange(nb) + 7] = np.maximum(pats >> 1, 1).astype(np.uint16) | 0x8000
    acc, q, e, ok, nbad = _twin_gpu(w)
    ref = oracle.make_twin(w)
    assert np.array_equal(e, ref.e) and np.array_equal(ok, ref.ok) and np.array_equal(q, ref.q)


def test_make_twin_amax_anywhere_in_its_block():
    # the largest element of each block at a random row and column (every lane position of the
    # encoder's row groups), ragged strips (the column count is not a multiple of 8 blocks), some
    # blocks rejected by a value with too many significant bits, some holding inf or NaN
    r = S.rng(3010)
    src = S.twin_source(3011, G=3, R=64, D=32 * 13)
    w = oracle.dequant_bf16(src["q"], src["e"]).copy()
    G, R, D = w.shape
    for g in range(G):
        for rb in range(R // 32):
            for cb in range(D // 32):
                i, j = rb * 32 + int(r.integers(0, 32)), cb * 32 + int(r.integers(0, 32))
                kind = int(r.integers(0, 10))
                if kind == 0:
                    w[g, i, j] = 0x3F81 | (w[g, i, j] & 0x8000)         # 8 significant bits
                elif kind == 1:
                    w[g, i, j] = 0x7F80 if r.integers(0, 2) else 0xFFC1  # inf or NaN
                elif kind == 2:
                    w[g, i, j] = 0x43E0                                   # 448 as the maximum
    acc, q, e, ok, nbad = _twin_gpu(w)
    ref = oracle.make_twin(w)
    assert np.array_equal(e, ref.e) and np.array_equal(ok, ref.ok)
    assert np.array_equal(q, ref.q)
    assert nbad == int((ref.ok == 0).sum()) and acc == ref.accepted


def test_pad_k_weight_and_input_bitwise():
    d = S.shared_down(3100, M=6, N=256, K=576)
    e = oracle.scales_from_f32(d["scales"], 256, 576)[None]
    qp, ep = B.bsfp8_pad_k_weight(to_gpu_u8(d["q"]), to_gpu_u8(e), 640)
    rq, re_ = oracle.pad_k_weight(d["q"], e, 640)
    assert np.array_equal(qp.cpu().numpy(), rq) and np.array_equal(ep.cpu().numpy(), re_)
    xp = B.bsfp8_pad_k_input(to_gpu_bf16(d["x"]), 1, 576, 640)
    assert np.array_equal(bf16_bits(xp), oracle.pad_k_input(d["x"], 1, 576, 640))
    # grouped and strided input, vector and scalar kernels
    x = S.bf16_normal(S.rng(3101), (3, 2 * 96 + 8))
    for cols in (2 * 96 + 8, 2 * 96 + 3):
        xt = to_gpu_bf16(x)[:, :cols] if cols <= x.shape[1] else None
        xt = to_gpu_bf16(np.ascontiguousarray(x[:, :cols]))
        got = B.bsfp8_pad_k_input(xt, 2, 96, 160)
        assert np.array_equal(bf16_bits(got), oracle.pad_k_input(x[:, :cols], 2, 96, 160))


def test_dequant_all_codes_all_exponents_bitwise():
    codes = np.array([c if c not in (0x7F, 0xFF) else 0 for c in range(256)], dtype=np.uint8)
    q = np.broadcast_to(codes, (255 * 32, 256)).reshape(1, 255 * 32, 256).copy()
    e = np.repeat(np.arange(255, dtype=np.uint8), 8).reshape(1, 255, 8)   # block row r has byte r
    got = bf16_bits(B.bsfp8_dequant(to_gpu_u8(q), to_gpu_u8(e)))
    assert np.array_equal(got, oracle.dequant_bf16(q, e))


def test_dequant_over_several_launches_bitwise():
    """More than 2^30 codes: the library dequantises in row ranges of under 2^30 codes (its indices
    are 32-bit); rows on both sides of each range boundary, and the last rows, equal the oracle."""
    K = 1 << 14
    N = (1 << 16) + 96                      # 65632 rows: the first range holds 65536 of them
    g = torch.Generator(device="cuda").manual_seed(3300)
    q = torch.randint(0, 256, (1, N, K), dtype=torch.uint8, device="cuda", generator=g)
    q[q == 0x7F] = 0
    q[q == 0xFF] = 0
    e = torch.randint(110, 140, (1, N // 32, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    w = B.bsfp8_dequant(q, e)
    torch.cuda.synchronize()
    for r0 in (0, 65504, 65536, N - 32):
        qs = q[:, r0:r0 + 32].cpu().numpy()
        es = e[:, r0 // 32:r0 // 32 + 1].cpu().numpy()
        got = bf16_bits(w[:, r0:r0 + 32])
        assert np.array_equal(got, oracle.dequant_bf16(qs, es)), r0
    del w, q


def test_dequant_round_trip_of_twin():
    src = S.twin_source(3200, G=4, R=128, D=256)
    w = oracle.dequant_bf16(src["q"], src["e"])
    t = B.bsfp8_make_twin(to_gpu_bf16(w))
    assert t.accepted
    back = bf16_bits(B.bsfp8_dequant(t.q, t.e))
    assert np.array_equal(back, w)


def test_pad_invariance_gemm_bitwise_full_shape():
    # shared-expert down_proj at its real size: K = 576 against K zero-padded to 640 (zero codes,
    # unit exponents, zero input tail) must give identical Y bits
    d = S.shared_down(1000, M=6, N=5120, K=576)
    e = B.bsfp8_scales_from_f32(torch.from_numpy(d["scales"]).cuda())[None]
    q = to_gpu_u8(d["q"])
    x = to_gpu_bf16(d["x"])
    y576 = B.bsfp8_gemm(x, q, e)
    qp, ep = B.bsfp8_pad_k_weight(q, e, 640)
    xp = B.bsfp8_pad_k_input(x, 1, 576, 640)
    y640 = B.bsfp8_gemm(xp, qp, ep)
    torch.cuda.synchronize()
    assert torch.equal(y576.view(torch.int16), y640.view(torch.int16))
    # the pad exponent byte does not matter (zero codes times any factor are zero)
    ep2 = ep.clone()
    ep2[:, :, 18:] = 200
    assert torch.equal(B.bsfp8_gemm(xp, qp, ep2).view(torch.int16), y576.view(torch.int16))
    check_bf16(bf16_bits(y576), d["x"], 1, 5120, 576, d["q"], e.cpu().numpy())
