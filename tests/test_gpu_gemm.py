"""GPU parity of the block-scaled fp8 GEMM against the CPU oracle, through the C ABI.

Sizes here span several workgroup tiles, m-blocks, splits and ragged K tails while the float64
oracle still finishes in seconds; full workload sizes are in test_gpu_workloads.py."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import synthetic as S
from parity import bf16_bits, check_bf16, check_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _inputs(seed, M, G, N, K, ldx=None, elo=110, ehi=130):
    r = S.rng(seed)
    ldx = ldx or G * K
    x = S.bf16_normal(r, (M, ldx))
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), elo, ehi)
    return x, q, e


def _run(entry, x, q, e, G, K, split_k=0, out_dtype="bf16"):
    xt = to_gpu_bf16(x)
    y = getattr(B, entry)(xt, to_gpu_u8(q), to_gpu_u8(e), split_k=split_k, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


SHAPES = [
    (1, 1, 32, 32), (2, 2, 64, 160), (6, 1, 96, 576), (8, 2, 128, 1024), (5, 3, 64, 416),
    (16, 1, 256, 2304), (7, 2, 192, 4096),
]


@pytest.mark.parametrize("M,G,N,K", SHAPES)
@pytest.mark.parametrize("entry", ["bsfp8_gemm_small", "bsfp8_gemm"])
def test_gemm_small_parity(entry, M, G, N, K):
    x, q, e = _inputs(100 + M + K, M, G, N, K)
    y = _run(entry, x, q, e, G, K)
    assert y.shape == (M, G, N)
    check_bf16(bf16_bits(y), x, G, N, K, q, e)


@pytest.mark.parametrize("M,G,N,K", [(9, 2, 128, 1024), (17, 1, 64, 800), (33, 2, 128, 640),
                                     (64, 1, 96, 4096), (100, 2, 64, 1152), (192, 1, 128, 512),
                                     (256, 1, 64, 256)])
def test_gemm_mid_parity(M, G, N, K):
    x, q, e = _inputs(200 + M + K, M, G, N, K)
    y = _run("bsfp8_gemm_mid", x, q, e, G, K)
    check_bf16(bf16_bits(y), x, G, N, K, q, e)


@pytest.mark.parametrize("split_k", [1, 2, 3, 8, 64])
def test_explicit_split_k(split_k):
    M, G, N, K = 6, 2, 128, 2048
    x, q, e = _inputs(300 + split_k, M, G, N, K)
    y = _run("bsfp8_gemm", x, q, e, G, K, split_k=split_k)
    check_bf16(bf16_bits(y), x, G, N, K, q, e)


@pytest.mark.parametrize("M,G,N,K", [(6, 1, 64, 5120), (40, 2, 64, 4608), (12, 1, 32, 8192),
                                     (40, 1, 32, 8320)])
def test_one_split_over_a_long_k(M, G, N, K):
    """split_k=1 with more chunks than a one-pass kernel holds: the plan falls back to the staged
    kernel, which walks the whole K range in passes, or (33..64 rows, K in whole chunks, at most
    64 of them) keeps the slab kernel, which walks any K range in slabs."""
    p = B.bsfp8_plan_info(M, G, N, K, split_k=1)
    kind = B.bsfp8_config_info(p["cfg"])["kind"]
    assert p["splits"] == 1 and kind in (0, 5)
    assert (kind == 5) == (33 <= M <= 64 and K % 128 == 0 and K <= 8192)
    x, q, e = _inputs(350 + M, M, G, N, K)
    y = _run("bsfp8_gemm", x, q, e, G, K, split_k=1)
    check_bf16(bf16_bits(y), x, G, N, K, q, e)


def _takes_ragged_k(cfg):
    """Whether a configuration accepts K that is not a multiple of 128 (the call is refused before
    any launch when it does not)."""
    x = torch.zeros((1, 800), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((1, 256, 800), dtype=torch.uint8, device="cuda")
    e = torch.full((1, 8, 25), 127, dtype=torch.uint8, device="cuda")
    try:
        B.bsfp8_gemm_config(x, q, e, cfg, 7)
    except B.BsfpError as err:
        assert err.status in (B.EINVAL, B.ESHAPE)
        return False
    torch.cuda.synchronize()
    return True


@pytest.mark.parametrize("M,K", [(1, 32), (6, 96), (6, 576), (8, 800), (3, 1120), (16, 2080)])
def test_ragged_k_decode_equals_the_register_kernel_and_the_padded_k(M, K):
    """K that is not whole 128-wide chunks at decode row counts: the plan takes the decode
    kernel's ragged instance, whose result equals bitwise the one-pass register kernel with the
    same waves and chunks and the decode kernel on K zero-padded to whole chunks (the same fp32
    chains with exact zeros added), and meets the parity rule against the oracle."""
    G, N = 2, 128
    x, q, e = _inputs(700 + K + M, M, G, N, K)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    plan = B.bsfp8_plan_info(M, G, N, K)
    info = B.bsfp8_config_info(plan["cfg"])
    print(f"M={M} K={K} plan {plan} {info}", flush=True)
    assert info["kind"] == 4
    y = B.bsfp8_gemm(xt, qt, et)
    direct = 21 if (info["NWK"], info["CW"]) == (4, 2) else 20    # the register kernel's twins
    yd = B.bsfp8_gemm_config(xt, qt, et, direct, plan["cps"])
    Kp = -(-K // 128) * 128
    qp, ep = B.bsfp8_pad_k_weight(qt, et, Kp)
    yp = B.bsfp8_gemm(B.bsfp8_pad_k_input(xt, G, K, Kp), qp, ep)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yd.view(torch.int16))
    assert torch.equal(y.view(torch.int16), yp.view(torch.int16))
    print(check_bf16(bf16_bits(y), x, G, N, K, q, e), flush=True)


def test_every_kernel_configuration():
    """Each compiled configuration, with a few chunks-per-split values, on a shape with several
    m-blocks (where the tile is smaller than M), a ragged K tail (the tile, slab, LDS-staged
    register and aligned decode kernels take K in whole 128-wide chunks) and every N tile width."""
    N = 256
    for cfg in range(B.bsfp8_num_configs()):
        info = B.bsfp8_config_info(cfg)
        if info["row_scales"]:              # these read [G][N][K/32] exponents: test_gpu_row32.py
            continue
        # the XCD-grouped tile maps take G = 8 / (XCDs per group), every other configuration G = 2
        G = 8 // info["xcds_per_group"] if info["xcds_per_group"] else 2
        K = 768 if info["kind"] in (3, 4, 5, 6, 8) else 800
        if info["kind"] in (4, 6) and _takes_ragged_k(cfg):
            K = 800                         # a decode instance built for a ragged last chunk
        if info["kind"] == 7:               # exactly the workgroup's chunks, one split
            K = 128 * info["CW"] * info["NWK"]
        M = min(2 * info["BM"] - 3, 256)
        x, q, e = _inputs(400 + cfg, M, G, N, K)
        exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
        if info["kind"] in (1, 2, 4, 6, 8):  # one pass: chunks per split <= CW * NWK
            cps_list = sorted({1, 2, info["CW"] * info["NWK"]})
        elif info["kind"] == 7:
            cps_list = (K // 128,)
        elif info["kind"] == 5:             # splits on 4-chunk slab boundaries, a partial last slab
            cps_list = (4, (K + 127) // 128)
        else:                               # several splits, and one split over all the chunks
            cps_list = (1, 2, (K + 127) // 128)
        for cps in cps_list:
            print(f"cfg {cfg} {info} cps {cps} M {M}", flush=True)
            y = B.bsfp8_gemm_config(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e), cfg, cps)
            torch.cuda.synchronize()
            check_bf16(bf16_bits(y), x, G, N, K, q, e, exact=exact)


def test_xcd_grouped_instances_bitwise_equal_to_the_plain_map():
    """The XCD-grouped tile maps only change which workgroup computes which tile: every output
    equals the plain map's bit for bit (paired kernel at two groups, decode kernel at two and
    four groups), and a group count the map was not built for is refused."""
    pairs = [(110, 93, 2), (111, 109, 2), (112, 54, 2), (113, 54, 4)]
    K = 4096
    for new, base, G in pairs:
        ni = B.bsfp8_config_info(new)
        assert ni["xcds_per_group"] * G == 8
        N = 512
        for M in (1, 3, 6, 8):
            x, q, e = _inputs(900 + new + M, M, G, N, K, elo=118, ehi=122)
            xg, qg, eg = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
            for od in ("bf16", "f32"):
                print(f"cfg {new} vs {base} G {G} M {M} {od}", flush=True)
                a = B.bsfp8_gemm_config(xg, qg, eg, new, 32, out_dtype=od)
                b = B.bsfp8_gemm_config(xg, qg, eg, base, 32, out_dtype=od)
                torch.cuda.synchronize()
                it = torch.int32 if od == "f32" else torch.int16
                assert torch.equal(a.view(it), b.view(it)), (new, M, od)
        x, q, e = _inputs(990, 2, 1, N, K)             # one group: not the count the map serves
        with pytest.raises(B.BsfpError):
            B.bsfp8_gemm_config(to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e), new, 32)


def test_fp32_output():
    M, G, N, K = 12, 1, 256, 1536
    x, q, e = _inputs(500, M, G, N, K, elo=118, ehi=122)
    y = _run("bsfp8_gemm", x, q, e, G, K, out_dtype="f32")
    assert y.dtype == torch.float32
    check_f32(y.cpu().numpy(), x, G, N, K, q, e)


def test_integer_exact_inputs_are_bitwise():
    # small integers times integer-valued codes at factor 1: every partial sum is an exact fp32
    # integer, so any summation order must equal the oracle bit for bit
    M, G, N, K = 8, 2, 128, 1024
    r = S.rng(600)
    x = S.small_int_bf16(r, (M, G * K), -4, 4)
    vals = oracle.decode_e4m3(np.arange(256))
    codes = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] == int(vals[c])
                      and abs(vals[c]) <= 16], dtype=np.uint8)
    q = codes[r.integers(0, codes.size, (G, N, K))]
    e = np.full((G, N // 32, K // 32), 127, dtype=np.uint8)
    for entry, sk in (("bsfp8_gemm", 0), ("bsfp8_gemm", 3), ("bsfp8_gemm_mid", 0)):
        y = bf16_bits(_run(entry, x, q, e, G, K, split_k=sk))
        ref = oracle.gemm(x, G, N, K, q, e)
        nz = (ref & 0x7FFF) != 0
        assert np.array_equal(y[nz], ref[nz]), entry
        assert np.all((y[~nz] & 0x7FFF) == 0)


def test_one_hot_rows_give_the_weights_bitwise():
    M, G, N, K = 4, 2, 128, 640
    r = S.rng(601)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 110, 130)
    W = oracle.dequant_bf16(q, e)
    ks = [0, 129, 383, 639]
    for g in range(G):
        x = np.zeros((M, G * K), dtype=np.uint16)
        for m, k in enumerate(ks):
            x[m, g * K + k] = 0x3F80
        y = bf16_bits(_run("bsfp8_gemm", x, q, e, G, K))
        for m, k in enumerate(ks):
            want = W[g, :, k]
            nz = (want & 0x7FFF) != 0
            assert np.array_equal(y[m, g][nz], want[nz])
            assert np.all((y[m, 1 - g] & 0x7FFF) == 0)


def test_strided_and_3d_activation_layouts():
    M, G, N, K = 5, 2, 64, 256
    ldx = G * K + 24
    x, q, e = _inputs(700, M, G, N, K, ldx=ldx)
    xt = to_gpu_bf16(x)
    y2 = B.bsfp8_gemm(xt, to_gpu_u8(q), to_gpu_u8(e))          # [M, ldx] with ldx > G*K
    y3 = B.bsfp8_gemm(xt.as_strided((M, G, K), (ldx, K, 1)), to_gpu_u8(q), to_gpu_u8(e))
    torch.cuda.synchronize()
    assert torch.equal(y2, y3)
    check_bf16(bf16_bits(y2), x[:, : G * K], G, N, K, q, e)


def test_run_to_run_bitwise_determinism():
    M, G, N, K = 8, 2, 1024, 4096
    x, q, e = _inputs(800, M, G, N, K, elo=115, ehi=125)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    for sk in (0, 8, 32):
        ws = B.workspace(M, G, N, K, sk)
        first = B.bsfp8_gemm(xt, qt, et, split_k=sk, ws=ws)
        for _ in range(50):
            again = B.bsfp8_gemm(xt, qt, et, split_k=sk, ws=ws)
            assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    torch.cuda.synchronize()


def test_determinism_under_concurrent_load():
    M, G, N, K = 6, 2, 1024, 4096
    x, q, e = _inputs(801, M, G, N, K, elo=115, ehi=125)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    ref = B.bsfp8_gemm(xt, qt, et, split_k=8)
    side = torch.cuda.Stream()
    ws_main = B.workspace(M, G, N, K, 8)
    ws_side = B.workspace(M, G, N, K, 8)
    outs = []
    torch.cuda.synchronize()
    for i in range(20):
        with torch.cuda.stream(side):
            B.bsfp8_gemm(xt, qt, et, split_k=8, ws=ws_side)
        outs.append(B.bsfp8_gemm(xt, qt, et, split_k=8, ws=ws_main))
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_graph_replays_match_eager():
    M, G, N, K = 6, 2, 1024, 4096
    x, q, e = _inputs(802, M, G, N, K, elo=115, ehi=125)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    ws = B.workspace(M, G, N, K, 0)
    out = torch.empty((M, G, N), dtype=torch.bfloat16, device="cuda")
    eager = B.bsfp8_gemm(xt, qt, et, ws=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.bsfp8_gemm(xt, qt, et, ws=ws, out=out)          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.bsfp8_gemm(xt, qt, et, ws=ws, out=out)
    for i in range(5):
        out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        B.bsfp8_gemm(xt, qt, et, ws=ws)                    # eager work between replays
        torch.cuda.synchronize()


def test_empty_and_error_cases():
    G, N, K = 1, 64, 128
    q = torch.zeros((G, N, K), dtype=torch.uint8, device="cuda")
    e = torch.full((G, N // 32, K // 32), 127, dtype=torch.uint8, device="cuda")
    x0 = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    y0 = B.bsfp8_gemm(x0, q, e)
    assert y0.shape == (0, G, N)
    x = torch.zeros((17, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_gemm_small(x, q, e)                         # small path takes at most 16 rows
    assert ei.value.status == B.ESHAPE
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_gemm(torch.zeros((257, K), dtype=torch.bfloat16, device="cuda"), q, e)
    assert ei.value.status == B.ESHAPE
    q_bad = torch.zeros((G, N, 100), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_gemm(torch.zeros((2, 100), dtype=torch.bfloat16, device="cuda"), q_bad,
                     torch.zeros((1, 2, 3), dtype=torch.uint8, device="cuda"))
    assert ei.value.status == B.ESHAPE
    xs = torch.zeros((4, K + 3), dtype=torch.bfloat16, device="cuda")[:, :K]   # ldx % 8 != 0
    with pytest.raises(B.BsfpError) as ei:
        B.bsfp8_gemm(xs, q, e)
    assert ei.value.status == B.ESTRIDE
    e_odd = torch.full((e.numel() + 1,), 127, dtype=torch.uint8, device="cuda")[1:].view(e.shape)
    with pytest.raises(B.BsfpError) as ei:                  # exponent bytes not 4-byte aligned
        B.bsfp8_gemm(torch.zeros((4, K), dtype=torch.bfloat16, device="cuda"), q, e_odd)
    assert ei.value.status == B.ESTRIDE
    n = B.bsfp8_workspace_bytes(6, 2, 1024, 4096, 8)
    assert n > 0
    small_ws = torch.zeros(n - 16, dtype=torch.uint8, device="cuda")
    qq = torch.zeros((2, 1024, 4096), dtype=torch.uint8, device="cuda")
    ee = torch.full((2, 32, 128), 127, dtype=torch.uint8, device="cuda")
    x6 = torch.zeros((6, 8192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):                          # the binding sees the short buffer
        B.bsfp8_gemm(x6, qq, ee, split_k=8, ws=small_ws)
    y6 = torch.empty((6, 2, 1024), dtype=torch.bfloat16, device="cuda")
    full_ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    st = B.lib().bsfp8_gemm(B._ptr(x6), 8192, 6, 2, 1024, 4096, B._ptr(qq), B._ptr(ee), 8, B._ptr(full_ws), n - 16,
                            B._ptr(y6), B.OUT_BF16, B._stream(x6))   # the library sees a short ws_bytes
    assert st == B.EWORKSPACE
    torch.cuda.synchronize()


def test_outputs_overlapping_inputs_are_refused():
    """The C ABI refuses an output range that overlaps an input, the workspace or another output
    (checked on address ranges before any launch)."""
    G, N, K, M = 1, 64, 256, 4
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    base = buf.data_ptr()
    q = B._ptr(buf[: G * N * K])
    e = ctypes.c_void_p(base + 65536)
    x = ctypes.c_void_p(base + 131072)
    s = B._stream(buf)
    L = B.lib()
    y_over_x = ctypes.c_void_p(base + 131072 + 512)
    assert L.bsfp8_gemm(x, G * K, M, G, N, K, q, e, 0, None, 0, y_over_x, B.OUT_BF16, s) == B.EINVAL
    assert L.bsfp8_gemm(x, G * K, M, G, N, K, q, e, 0, None, 0, q, B.OUT_F32, s) == B.EINVAL
    y_ok = ctypes.c_void_p(base + 262144)
    assert L.bsfp8_gemm(x, G * K, M, G, N, K, q, e, 0, None, 0, y_ok, B.OUT_BF16, s) == B.OK
    yq, ys = ctypes.c_void_p(base + 393216), ctypes.c_void_p(base + 393216 + 64)   # ys inside yq
    ws = ctypes.c_void_p(base + 524288)
    assert L.bsfp8_gemm_mxfp8(x, G * K, M, G, N, K, q, e, 0, ws, 65536, yq, ys, s) == B.EINVAL
    assert L.bsfp8_quantize_mx(x, G * K, M, G * K, ctypes.c_void_p(base + 131072 + 256), ys, s) == B.EINVAL
    assert L.bsfp8_dequant(q, e, G, N, K, ctypes.c_void_p(base + 65536 - 64), s) == B.EINVAL
    torch.cuda.synchronize()


def test_binding_refuses_short_or_misplaced_buffers():
    """Every buffer the binding hands over is checked against the sizes the library will address
    (the C ABI cannot see allocation sizes), so a short or host buffer never reaches a kernel."""
    G, N, K, M = 2, 64, 256, 4
    q = torch.zeros((G, N, K), dtype=torch.uint8, device="cuda")
    e = torch.full((G, N // 32, K // 32), 127, dtype=torch.uint8, device="cuda")
    x = torch.zeros((M, G * K), dtype=torch.bfloat16, device="cuda")
    cases = [
        lambda: B.bsfp8_gemm(x, q, e, out=torch.empty((M, G, N - 1), dtype=torch.bfloat16, device="cuda")),
        lambda: B.bsfp8_gemm(x, q, e, out=torch.empty((M, G, N), dtype=torch.float32, device="cuda")),
        lambda: B.bsfp8_gemm(x, q, e[:, :1].contiguous()),
        lambda: B.bsfp8_gemm(x[:, : G * K - 8], q, e),
        lambda: B.bsfp8_gemm(x, q, e, split_k=2, ws=torch.zeros(8, dtype=torch.uint8)),   # host memory
        lambda: B.bsfp8_gemm(x, q, e, split_k=2, ws=torch.zeros(1 << 20, dtype=torch.float32, device="cuda")),
        lambda: B.bsfp8_gemm_config(x, q, e, 54, 2, out=torch.empty(1, dtype=torch.bfloat16, device="cuda")),
        lambda: B.bsfp8_gemm_row32(x, q, e),                  # block exponents where row exponents are due
        lambda: B.bsfp8_gemm_mxfp8(x, q, e, yq=torch.empty((M, G * N - 32), dtype=torch.uint8, device="cuda")),
        lambda: B.bsfp8_gemm_mxfp8(x, q, e, ws=torch.empty(4, dtype=torch.uint8, device="cuda")),
        lambda: B.bsfp8_quantize_mx(x, xs=torch.empty((M, 1), dtype=torch.uint8, device="cuda")),
        lambda: B.bsfp8_quantize_mx(x, L=G * K + 32),
        lambda: B.bsfp8_pad_k_input(x, G, K, K + 128, out=torch.empty((M, G * K), dtype=torch.bfloat16, device="cuda")),
        lambda: B.bsfp8_dequant(q, e, out=torch.empty((G, N, K - 1), dtype=torch.bfloat16, device="cuda")),
        lambda: B.bsfp8_pad_k_weight(q, e[:1].contiguous(), K + 128),
        lambda: B.bsfp8_scales_from_f32(torch.ones((2, 8), dtype=torch.float32, device="cuda"),
                                        exp_out=torch.empty(15, dtype=torch.uint8, device="cuda")),
    ]
    xq, xs = B.bsfp8_quantize_mx(x)
    cases += [
        lambda: B.bsfp8_gemm_mx(xq, xs, q, e, out=torch.empty(7, dtype=torch.bfloat16, device="cuda")),
        lambda: B.bsfp8_gemm_mx(xq[:, : G * K - 128], xs[:, : (G * K - 128) // 32], q, e),
        lambda: B.bsfp8_gemm_mx(xq, xs[:2], q, e),
        lambda: B.bsfp8_gemm_mx(xq, xs.cpu(), q, e),
    ]
    for i, case in enumerate(cases):
        with pytest.raises((ValueError, TypeError)):
            case()
            print(f"case {i} was not refused", flush=True)
    torch.cuda.synchronize()


def test_read_floor_reads_and_writes_in_bounds():
    """The measurement aid of the bench: the plain-read floor kernel reads the bytes it is given
    (and, with a slab, every workgroup its group's part of the slab), touches the sink only on its
    fixed constant, and with an output buffer writes every byte of it and nothing else (all-zero
    data fold to zero, so the written bytes are known)."""
    t = torch.zeros(8 * 1024 * 1024 + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.full((256,), 7, dtype=torch.int32, device="cuda")
    guard = torch.full((24576 + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    out = guard[:24576]
    slab = torch.zeros(2 * 49152, dtype=torch.uint8, device="cuda")
    B.bsfp8_read_floor(t, nwg=256, sink=sink)
    B.bsfp8_read_floor(t, nbytes=0, nwg=256, sink=sink)
    B.bsfp8_read_floor(t, nwg=256, sink=sink, out=out)
    B.bsfp8_read_floor(t, nwg=256, sink=sink, slab=slab, slab_groups=2)        # 48 KB per group
    B.bsfp8_read_floor(t, nbytes=0, nwg=256, sink=sink, slab=slab[:6912], slab_groups=1)
    # the slab spread over the steps of the share: one step (256 workgroups), six steps of twelve
    # loads per wave (16 workgroups), no share at all
    B.bsfp8_read_floor(t, nwg=256, sink=sink, slab=slab, slab_groups=2, interleave=True)
    B.bsfp8_read_floor(t, nwg=16, sink=sink[:16], slab=slab, slab_groups=2, interleave=True)
    B.bsfp8_read_floor(t, nbytes=0, nwg=256, sink=sink, slab=slab[:6912], slab_groups=1, interleave=True)
    guard[:24576].fill_(0xAB)
    B.bsfp8_read_floor(t, nwg=256, sink=sink, out=out, slab=slab, slab_groups=2)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
    assert bool((out == 0).all())
    guard[:24576].fill_(0xAB)
    B.bsfp8_read_floor(t, nwg=16, sink=sink[:16], out=out, slab=slab, slab_groups=2, interleave=True)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
    assert bool((out == 0).all())
    assert bool((guard[24576:] == 0xAB).all())
    with pytest.raises(B.BsfpError):
        B.bsfp8_read_floor(t, nwg=256, sink=sink, out=torch.empty(40, dtype=torch.uint8, device="cuda"))
