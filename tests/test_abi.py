"""CPU checks of the C ABI: the library loads, exports every symbol the headers declare, and its
host-side logic (status strings, plans, workspace sizes, argument checks that return before any
GPU work) behaves as documented. No kernel is launched here."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_skinny_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_scaled_fp8_skinny_amd import build
        build.build()
    return B.lib()


def _declared():
    names = set()
    for h in ("bsfp8.h", "bsfp8_tuning.h"):
        with open(os.path.join(ROOT, "include", h)) as f:
            names |= set(re.findall(r"BSFP8_API\s+[\w\s\*]*?\b(bsfp8_\w+)\s*\(", f.read()))
    return names


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 16
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in sorted(names):
        assert hasattr(raw, n), n
    assert set(B._SIGS) == names      # the binding covers exactly the declared entry points


def test_status_strings_and_version(lib):
    assert lib.bsfp8_abi_version() == 1
    for st in (0, 1, -1, -2, -3, -4, -5, -6):
        assert B.strerror(st) and B.strerror(st) != "unknown status"
    assert B.strerror(42) == "unknown status"


def test_workspace_and_plans(lib):
    # the headline decode shape: every chunk is owned by exactly one split
    p = B.bsfp8_plan_info(6, 2, 1024, 4096)
    assert p["splits"] * p["cps"] >= p["kchunks"] and p["workgroups"] >= 128
    ws = B.bsfp8_workspace_bytes(6, 2, 1024, 4096)
    assert ws >= p["splits"] * 6 * 2 * 1024 * 4 if p["splits"] > 1 else ws == 0
    # K and K padded inside the same 128-chunk count get the same fp32 chain for every output:
    # the same chunks per split and splits, and the same waves along K and chunks per wave (at
    # decode row counts both take the decode kernel: 576 its ragged instance, which reads zeros
    # past K)
    def chain(M, G, N, K):
        p = B.bsfp8_plan_info(M, G, N, K)
        info = B.bsfp8_config_info(p["cfg"])
        return (p["kchunks"], p["cps"], p["splits"], info["NWK"], info["CW"])
    for m in (1, 6, 8, 12, 16):
        assert chain(m, 1, 5120, 576) == chain(m, 1, 5120, 640)
    assert B.bsfp8_config_info(B.bsfp8_plan_info(6, 1, 5120, 640)["cfg"])["kind"] == 4
    assert B.bsfp8_config_info(B.bsfp8_plan_info(6, 1, 5120, 576)["cfg"])["kind"] == 4
    # explicit split_k
    p8 = B.bsfp8_plan_info(6, 2, 1024, 4096, split_k=8)
    assert p8["splits"] == 8
    assert B.bsfp8_workspace_bytes(6, 2, 1024, 4096, 1) == 0
    # the LM-head shape keeps one chunk map for every row count (per-row fp32 logits identical)
    plans = [B.bsfp8_plan_info(m, 1, 32768, 5120) for m in (16, 64, 128)]
    maps = {(p["kchunks"], p["cps"], p["splits"], B.bsfp8_config_info(p["cfg"])["NWK"]) for p in plans}
    assert len(maps) == 1
    for cfg in range(B.bsfp8_num_configs()):
        info = B.bsfp8_config_info(cfg)
        # weight tiles are whole 16-row MFMA tiles, or 8 rows: half tiles for row-scale twins, and
        # the paired decode kernel (kinds 6, 7), whose MFMA rows 8..15 carry the same rows' next chunk
        assert info["BM"] % 8 == 0 and info["threads"] % 64 == 0
        assert info["NB"] % 16 == 0 or ((info["row_scales"] or info["kind"] in (6, 7)) and info["NB"] % 8 == 0)


def test_plan_is_valid_for_every_shape_class(lib):
    """The built-in plan picks a compiled configuration that accepts the shape for every row count
    1..256, N and K multiples of 32 (ragged and whole 128-chunk K, narrow and wide weights), G in
    1, 2, 4, with and without an explicit split, and every chunk is owned by exactly one split."""
    Ks = [32, 96, 128, 576, 640, 800, 2048, 4096, 5120, 8192]
    Ns = [32, 96, 128, 1024, 5120, 16384, 32768]
    for M in list(range(1, 33)) + [48, 63, 64, 65, 96, 127, 128, 129, 160, 192, 193, 224, 256]:
        for G in (1, 2, 4):
            for N in Ns:
                if G * N > 65536:
                    continue
                for K in Ks:
                    for split_k in (0, 1, 3):
                        p = B.bsfp8_plan_info(M, G, N, K, split_k=split_k)
                        kch = (K + 127) // 128
                        assert p["kchunks"] == kch
                        assert (p["splits"] - 1) * p["cps"] < kch <= p["splits"] * p["cps"], (M, G, N, K, split_k, p)
                        assert p["mblocks"] * p["BM"] >= M and N % p["NB"] == 0
                        info = B.bsfp8_config_info(p["cfg"])
                        if info["kind"] in (3, 5, 8) or (info["kind"] == 4 and info["row_scales"]):
                            assert K % 128 == 0     # the decode kernel takes a ragged last chunk
                        if info["kind"] == 5 and p["splits"] > 1:
                            assert p["cps"] % 4 == 0
                        if split_k:
                            assert p["splits"] == -(-kch // -(-kch // split_k))
                        ws = B.bsfp8_workspace_bytes(M, G, N, K, split_k)
                        assert (ws == 0) == (p["splits"] == 1) or ws > 0


def test_argument_checks_return_before_gpu_work(lib):
    null = ctypes.c_void_p(0)
    G = lib.bsfp8_gemm
    # bad out dtype, bad shapes, split_k out of range, null pointers, bad ldx: all host checks
    assert G(null, 64, 1, 1, 64, 64, null, null, 0, null, 0, null, 7, null) == B.EINVAL
    assert G(null, 64, 1, 1, 64, 40, null, null, 0, null, 0, null, 0, null) == B.ESHAPE
    assert G(null, 64, 300, 1, 64, 64, null, null, 0, null, 0, null, 0, null) == B.ESHAPE
    assert G(null, 64, 1, 1, 64, 64, null, null, 65, null, 0, null, 0, null) == B.EINVAL
    assert G(null, 64, 1, 1, 64, 64, null, null, 0, null, 0, null, 0, null) == B.EINVAL
    assert lib.bsfp8_gemm_small(null, 64, 17, 1, 64, 64, null, null, 0, null, 0, null, 0, null) == B.ESHAPE
    assert G(null, 64, 0, 1, 64, 64, null, null, 0, null, 0, null, 0, null) == B.OK   # empty: no-op
    fake = ctypes.c_void_p(4096)
    assert G(fake, 60, 1, 1, 64, 64, fake, fake, 0, null, 0, fake, 0, null) == B.ESTRIDE
    assert G(fake, 68, 1, 1, 64, 64, fake, fake, 0, null, 0, fake, 0, null) == B.ESTRIDE
    assert G(ctypes.c_void_p(4104), 64, 1, 1, 64, 64, fake, fake, 0, null, 0, fake, 0, null) == B.ESTRIDE
    # a split plan without its workspace (distinct, non-overlapping buffers)
    xa, qa, ea, ya = (ctypes.c_void_p(i << 32) for i in (1, 2, 3, 4))
    assert G(xa, 8192, 6, 2, 1024, 4096, qa, ea, 8, null, 0, ya, 0, null) == B.EWORKSPACE
    # outputs overlapping an input, the workspace or another output
    assert G(xa, 8192, 6, 2, 1024, 4096, qa, ea, 0, null, 0, ctypes.c_void_p((1 << 32) + 4096), 0, null) == B.EINVAL
    assert G(xa, 8192, 6, 2, 1024, 4096, qa, ea, 0, null, 0, ctypes.c_void_p((3 << 32) - 16), 1, null) == B.EINVAL
    wsa = ctypes.c_void_p(5 << 32)
    assert G(xa, 8192, 6, 2, 1024, 4096, qa, ea, 8, wsa, 1 << 24, ctypes.c_void_p((5 << 32) + 256), 0, null) == B.EINVAL
    assert lib.bsfp8_gemm_mxfp8(xa, 8192, 6, 2, 1024, 4096, qa, ea, 0, wsa, 1 << 24, ya,
                                ctypes.c_void_p((4 << 32) + 1024), null) == B.EINVAL      # ys inside yq
    assert lib.bsfp8_quantize_mx(xa, 8192, 6, 8192, ctypes.c_void_p((1 << 32) + 8192), ya, null) == B.EINVAL
    assert lib.bsfp8_reduce_quantize_mx(xa, 2, 6, 1024, 0, ya, ctypes.c_void_p((1 << 32) + 64), null) == B.EINVAL
    assert lib.bsfp8_dequant(qa, ea, 1, 64, 64, ctypes.c_void_p((2 << 32) + 16), null) == B.EINVAL
    assert lib.bsfp8_pad_k_input(xa, 64, 2, 1, 64, 128, ctypes.c_void_p((1 << 32) + 64), null) == B.EINVAL
    assert lib.bsfp8_pad_k_weight(qa, ea, 1, 64, 64, 128, ya, ctypes.c_void_p((3 << 32) + 2), null) == B.EINVAL
    # the entry point without a workspace: the same host checks, and a plan beyond its static
    # scratch is refused before the scratch is looked up or anything is enqueued
    NA = lib.bsfp8_gemm_no_alloc
    assert NA(null, 64, 1, 1, 64, 64, null, null, 0, null, 7, null) == B.EINVAL
    assert NA(null, 64, 300, 1, 64, 64, null, null, 0, null, 0, null) == B.ESHAPE
    assert NA(null, 64, 0, 1, 64, 64, null, null, 0, null, 0, null) == B.OK
    assert NA(fake, 60, 1, 1, 64, 64, fake, fake, 0, fake, 0, null) == B.ESTRIDE
    assert NA(xa, 4096, 256, 1, 8192, 4096, qa, ea, 8, ya, 0, null) == B.EWORKSPACE
    assert B.bsfp8_workspace_bytes(256, 1, 8192, 4096, 8) > B.NO_ALLOC_SCRATCH_BYTES
    assert NA(xa, 8192, 6, 2, 1024, 4096, qa, ea, 0, ctypes.c_void_p((1 << 32) + 4096), 0, null) == B.EINVAL
    hdr = open(os.path.join(ROOT, "include", "bsfp8.h")).read()
    m = re.search(r"#define BSFP8_NO_ALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NO_ALLOC_SCRATCH_BYTES
    # the floor kernel's checks: a sink, an output buffer when output bytes are asked for, 16-byte
    # alignment and a multiple of 16 bytes, and no overlap with what it reads
    F = lib.bsfp8_read_floor
    # F(p, bytes, nwg, slab, slab_bytes, slab_groups, flags, sink, out, out_bytes, stream)
    assert F(xa, 1024, 0, null, 0, 1, 0, ya, null, 0, null) == B.EINVAL
    assert F(xa, 1024, 4, null, 0, 1, 0, null, null, 0, null) == B.EINVAL
    assert F(xa, 1024, 4, null, 0, 1, 0, ya, null, 64, null) == B.EINVAL
    assert F(xa, 1024, 4, null, 0, 1, 2, ya, null, 0, null) == B.EINVAL     # unknown flag
    assert F(ctypes.c_void_p((1 << 32) + 8), 1024, 4, null, 0, 1, 0, ya, null, 0, null) == B.ESTRIDE
    assert F(xa, 1024, 4, null, 0, 1, 0, ya, ctypes.c_void_p((4 << 32) + 4096 + 8), 64, null) == B.ESTRIDE
    assert F(xa, 1024, 4, null, 0, 1, 0, ya, ctypes.c_void_p((4 << 32) + 4096), 40, null) == B.ESTRIDE
    assert F(xa, 1 << 31, 4, null, 0, 1, 0, ya, null, 0, null) == B.ESHAPE
    assert F(xa, 1024, 4, null, 0, 1, 0, ya, ctypes.c_void_p((1 << 32) + 512), 64, null) == B.EINVAL
    # the slab: present when it has bytes, 1..nwg groups, aligned, a multiple of 16 bytes, under
    # 2^31 bytes in all, and no output over it
    sl = ctypes.c_void_p(5 << 32)
    assert F(xa, 1024, 4, null, 64, 1, 0, ya, null, 0, null) == B.EINVAL
    assert F(xa, 1024, 4, sl, 64, 0, 0, ya, null, 0, null) == B.EINVAL
    assert F(xa, 1024, 4, sl, 64, 5, 0, ya, null, 0, null) == B.EINVAL
    assert F(xa, 1024, 4, ctypes.c_void_p((5 << 32) + 8), 64, 1, 0, ya, null, 0, null) == B.ESTRIDE
    assert F(xa, 1024, 4, sl, 40, 1, 0, ya, null, 0, null) == B.ESTRIDE
    assert F(xa, 1024, 4, sl, 1 << 30, 2, 0, ya, null, 0, null) == B.ESHAPE
    assert F(xa, 1024, 4, sl, 4096, 2, 0, ya, ctypes.c_void_p((5 << 32) + 4096), 64, null) == B.EINVAL
    assert F(xa, 1024, 4, sl, 4096, 2, 0, ctypes.c_void_p((5 << 32) + 64), null, 0, null) == B.EINVAL
    bad = ctypes.c_int64(0)
    assert lib.bsfp8_make_twin(null, 1, 33, 32, null, null, null, ctypes.byref(bad), null) == B.ESHAPE
    # the asynchronous encoder: a device counter, 8-byte aligned, outside w and the outputs
    TA = lib.bsfp8_make_twin_async
    wa, qa, ea = ctypes.c_void_p(6 << 32), ctypes.c_void_p(7 << 32), ctypes.c_void_p(8 << 32)
    cnt = ctypes.c_void_p(9 << 32)
    assert TA(wa, 1, 33, 32, qa, ea, null, cnt, null) == B.ESHAPE
    assert TA(wa, 1, 32, 32, qa, ea, null, null, null) == B.EINVAL
    assert TA(wa, 1, 32, 32, qa, ea, null, ctypes.c_void_p((9 << 32) + 4), null) == B.EINVAL
    assert TA(wa, 1, 32, 32, qa, ea, null, ctypes.c_void_p((6 << 32) + 64), null) == B.EINVAL   # inside w
    assert TA(wa, 1, 32, 32, qa, ea, null, ctypes.c_void_p((7 << 32) + 8), null) == B.EINVAL    # inside q
    assert TA(ctypes.c_void_p((6 << 32) + 8), 1, 32, 32, qa, ea, null, cnt, null) == B.ESTRIDE
    assert TA(wa, 0, 32, 32, qa, ea, null, cnt, null) == B.OK                                   # nothing to do
    assert lib.bsfp8_pad_k_weight(null, null, 1, 32, 64, 48, null, null, null) == B.ESHAPE
    assert lib.bsfp8_pad_k_input(null, 10, 1, 1, 32, 64, null, null) == B.ESTRIDE
    assert lib.bsfp8_dequant(null, null, 1, 32, 40, null, null) == B.ESHAPE
    assert lib.bsfp8_dequant(null, null, 1, 32, (1 << 24) + 32, null, null) == B.ESHAPE
    assert lib.bsfp8_scales_from_f32(null, -1, 2, null, ctypes.byref(bad), null) == B.ESHAPE


def test_mx_argument_checks_and_plans(lib):
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(4096)
    Q, X = lib.bsfp8_quantize_mx, lib.bsfp8_gemm_mx
    assert Q(null, 64, 0, 64, null, null, null) == B.OK                     # empty: no-op
    assert Q(null, 64, 2, 48, null, null, null) == B.ESHAPE                 # L not a multiple of 32
    assert Q(fake, 32, 2, 64, fake, fake, null) == B.ESTRIDE                # ldx < L
    assert Q(ctypes.c_void_p(4104), 64, 2, 64, fake, fake, null) == B.ESTRIDE   # x not 16-byte aligned
    assert Q(null, 64, 2, 64, null, null, null) == B.EINVAL
    # gemm_mx(xq, xs, ldq, M, G, N, K, q, e, y, out, stream)
    assert X(null, null, 256, 0, 1, 64, 256, null, null, null, 0, null) == B.OK     # empty: no-op
    assert X(null, null, 256, 1, 1, 64, 256, null, null, null, 9, null) == B.EINVAL  # out dtype
    assert X(fake, fake, 192, 1, 1, 64, 192, fake, fake, fake, 0, null) == B.ESHAPE  # K % 128
    assert X(fake, fake, 256, 257, 1, 64, 256, fake, fake, fake, 0, null) == B.ESHAPE  # M > 256
    assert X(fake, fake, 8320, 1, 1, 64, 8320, fake, fake, fake, 0, null) == B.ESHAPE  # K > 8192
    assert X(fake, fake, 320, 1, 1, 64, 256, fake, fake, fake, 0, null) == B.ESTRIDE   # ldq % 128
    assert X(fake, fake, 128, 1, 1, 64, 256, fake, fake, fake, 0, null) == B.ESTRIDE   # ldq < G*K
    assert X(fake, ctypes.c_void_p(4098), 256, 1, 1, 64, 256, fake, fake, fake, 0, null) == B.ESTRIDE
    assert X(null, fake, 256, 1, 1, 64, 256, fake, fake, fake, 0, null) == B.EINVAL
    # the plan picks a compiled configuration whose weight tile divides N, for every row count
    n = B.bsfp8_mx_num_configs()
    for M in range(1, 257):
        for G, N in ((2, 1024), (1, 32768), (1, 5120), (4, 1024), (1, 96), (1, 32)):
            cfg = B.bsfp8_mx_plan(M, G, N)
            assert 0 <= cfg < n and N % B.bsfp8_mx_config_info(cfg)["NB"] == 0, (M, G, N, cfg)
    assert lib.bsfp8_mx_plan(0, 1, 64) == B.ESHAPE


def test_row32_plans_and_checks(lib):
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(4096)
    X = lib.bsfp8_gemm_row32
    assert X(null, 128, 0, 1, 64, 128, null, null, 0, null, 0, null, 0, null) == B.OK          # empty
    assert X(fake, 256, 17, 1, 64, 256, fake, fake, 0, null, 0, fake, 0, null) == B.ESHAPE     # M > 16
    assert X(fake, 192, 2, 1, 64, 192, fake, fake, 0, null, 0, fake, 0, null) == B.ESHAPE     # K % 128
    bad = ctypes.c_int64(0)
    assert lib.bsfp8_make_twin_row32(null, 1, 2, 48, null, null, null, ctypes.byref(bad), null) == B.ESHAPE
    # the page's shape (K = 5120, 40 chunks) runs in one pass: no workspace
    for M in (1, 6, 16):
        assert B.bsfp8_workspace_bytes_row32(M, 1, 1280, 5120) == 0
    # a longer K is split over workgroups and needs exchange slots
    assert B.bsfp8_workspace_bytes_row32(6, 1, 1280, 8192) > 0
    # 32x32 configurations are refused on the row-scale entry and vice versa
    rs = [c for c in range(B.bsfp8_num_configs()) if B.bsfp8_config_info(c)["row_scales"]]
    assert rs
    assert lib.bsfp8_gemm_row32_config(fake, 256, 2, 1, 64, 256, fake, fake, 54, 2, null, 0, fake, 0, null) == B.EINVAL
    assert lib.bsfp8_gemm_config(fake, 256, 2, 1, 64, 256, fake, fake, rs[0], 2, null, 0, fake, 0, null) == B.EINVAL


def test_mxfp8_epilogue_checks_and_plans(lib):
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(4096)
    R = lib.bsfp8_reduce_quantize_mx
    # (part, S, M, L, order, yq, ys, stream)
    assert R(fake, 1, 2, 64, 2, fake, fake, null) == B.EINVAL                   # order
    assert R(fake, 0, 2, 64, 0, fake, fake, null) == B.EINVAL                   # S < 1
    assert R(fake, 65, 2, 64, 0, fake, fake, null) == B.EINVAL                  # S > 64
    assert R(fake, 1, 2, 48, 0, fake, fake, null) == B.ESHAPE                   # L % 32
    assert R(fake, 1, 2, 0, 0, fake, fake, null) == B.ESHAPE
    assert R(null, 1, 0, 64, 1, null, null, null) == B.OK                       # empty: no-op
    assert R(null, 1, 2, 64, 1, fake, fake, null) == B.EINVAL
    assert R(ctypes.c_void_p(4100), 1, 2, 64, 1, fake, fake, null) == B.ESTRIDE
    assert R(fake, 1, 2, 64, 1, ctypes.c_void_p(4100), fake, null) == B.ESTRIDE
    # the epilogue GEMM runs bsfp8_gemm's plan, except where that is the paired decode kernel
    # (8-row tiles, a quarter of an MX block): there it keeps the 16-row decode plan, whose fused
    # form quantises whole blocks; its workspace holds one fp32 copy per split
    for M, G, N, K, sk in ((6, 2, 1024, 4096, 0), (6, 2, 1024, 4096, 4), (64, 2, 1024, 4096, 0),
                           (16, 1, 32768, 5120, 0), (16, 1, 32768, 5120, 2), (6, 1, 5120, 576, 0)):
        p3 = B.bsfp8_plan_info(M, G, N, K, split_k=sk, path=3)
        p2 = B.bsfp8_plan_info(M, G, N, K, split_k=sk, path=2)
        if B.bsfp8_config_info(p2["cfg"])["kind"] in (6, 7):
            assert B.bsfp8_config_info(p3["cfg"])["kind"] == 4 and p3["splits"] == p2["splits"]
        else:
            assert p3 == p2
        assert B.bsfp8_workspace_bytes_mxfp8(M, G, N, K, sk) == p3["splits"] * M * G * N * 4
        assert B.bsfp8_workspace_bytes_mxfp8_config(M, G, N, K, p3["cfg"], p3["cps"]) == p3["splits"] * M * G * N * 4
    assert B.bsfp8_workspace_bytes_mxfp8(0, 2, 1024, 4096, 0) == 0
    X = lib.bsfp8_gemm_mxfp8
    # (x, ldx, M, G, N, K, q, e, split_k, ws, ws_bytes, yq, ys, stream)
    assert X(null, 64, 0, 1, 64, 64, null, null, 0, null, 0, null, null, null) == B.OK
    assert X(fake, 64, 1, 1, 64, 64, fake, fake, 0, fake, 1 << 20, fake, null, null) == B.EINVAL   # ys
    assert X(fake, 64, 1, 1, 64, 64, fake, fake, 0, fake, 16, fake, fake, null) == B.EWORKSPACE    # ws small
    assert X(fake, 64, 1, 1, 64, 64, fake, fake, 0, null, 0, fake, fake, null) == B.EWORKSPACE
    assert X(fake, 64, 1, 1, 64, 64, fake, fake, 0, fake, 1 << 20, ctypes.c_void_p(4097), fake, null) == B.ESTRIDE
    assert X(fake, 64, 1, 1, 64, 40, fake, fake, 0, fake, 1 << 20, fake, fake, null) == B.ESHAPE
    rs = [c for c in range(B.bsfp8_num_configs()) if B.bsfp8_config_info(c)["row_scales"]]
    assert lib.bsfp8_gemm_mxfp8_config(fake, 256, 2, 1, 64, 256, fake, fake, rs[0], 2, fake, 1 << 20, fake, fake,
                                       null) == B.EINVAL
