"""GPU parity at the edges of the exponent range and of the number formats, through every kind of
GEMM kernel, plus the split-K plans the configurations name at their full sizes.

* Exponent bytes 0..3 (block factors 2^-127..2^-124): the rebuilt weights are bf16 subnormals or
  round to them (the oracle rounds the exact product once, RNE; page
  "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py", kernel _wo_a_partial_w8 rebuilds the tile
  as bf16 of fp32(code) * 2^(b-127)). Subnormal weights must reach the MFMA unflushed.
* Exponent bytes 246, 250 and 254 (factors 2^119..2^127): the codes of those blocks are capped so
  that the rebuilt weights stay finite, and the activations are scaled down so that no fp32 sum
  overflows.
* A rebuilt weight beyond the bf16 range is +-inf, as the oracle's rounding says; exponent byte
  255 makes every output of its block rows NaN, and so does an e4m3 NaN code for its weight row
  (the header's promise).
* The twin of a block of bf16 subnormals (exponent byte 0) used in a GEMM.
* The wo_a configurations' own splits at full size (split-K 8 at 2..8 rows; 4 and 2 at 16 and 32
  rows, as the mid table of the page sets them), against the oracle.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import oracle
import synthetic as S
from parity import bf16_bits, check_bf16, check_bf16_exact, check_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _edge_inputs(seed, M, G, N, K, kind):
    r = S.rng(seed)
    if kind == "tiny":
        e, cls = S.edge_exponent_bytes(r, G, N, K, S.TINY_BYTES)
        q = S.e4m3_codes(r, (G, N, K))
        x = S.bf16_normal(r, (M, G * K))
    else:
        e, cls = S.edge_exponent_bytes(r, G, N, K, S.LARGE_BYTES)
        q = S.e4m3_codes(r, (G, N, K))
        # the largest exponent field per block that keeps code * 2^(b-127) below 2^128
        fmax = np.minimum(15, 261 - e.astype(np.int64))
        q = S.cap_code_exponent_field(q, np.repeat(np.repeat(fmax, 32, axis=1), 32, axis=2))
        x = S.bf16_normal(r, (M, G * K), scale=2.0 ** -40)
    return x, q, e, cls


def _check_both(y, y32, x, G, N, K, q, e):
    exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    assert np.isfinite(exact).all()
    st = check_bf16(bf16_bits(y), x, G, N, K, q, e, exact=exact)
    check_f32(y32.cpu().numpy(), x, G, N, K, q, e, exact=exact)
    assert torch.equal(y.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    return st


def _takes_ragged_k(cfg):
    """Whether a configuration accepts K that is not a multiple of 128 (others refuse the call
    before any launch)."""
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


def _kinds():
    """One configuration per distinct kernel (kind, waves, chunks, tile), 32x32 exponents."""
    out, seen = [], set()
    for cfg in range(B.bsfp8_num_configs()):
        info = B.bsfp8_config_info(cfg)
        if info["row_scales"]:
            continue
        key = (info["kind"], info["BM"], info["NB"], info["NWK"], info["CW"])
        if key in seen:
            continue
        seen.add(key)
        out.append(cfg)
    return out


@pytest.mark.parametrize("kind", ["tiny", "large"])
def test_extreme_exponent_bytes_every_kernel(kind):
    """Every kernel configuration on weights whose block rows hold only extreme exponent bytes,
    a half-and-half mix with ordinary ones, or only ordinary ones; bf16 and fp32 outputs."""
    G, N = 2, 256
    for cfg in _kinds():
        info = B.bsfp8_config_info(cfg)
        K = 768 if info["kind"] in (3, 4, 5, 6, 8) and not _takes_ragged_k(cfg) else 800
        if info["kind"] == 7:                          # exactly the workgroup's chunks
            K = 128 * info["CW"] * info["NWK"]
        M = min(2 * info["BM"] - 3, 256)
        x, q, e, _ = _edge_inputs(9100 + cfg + (0 if kind == "tiny" else 500), M, G, N, K, kind)
        cps = info["CW"] * info["NWK"] if info["kind"] in (1, 2, 4, 6, 7, 8) else (K + 127) // 128
        print(f"{kind} cfg {cfg} {info} M {M} K {K} cps {cps}", flush=True)
        xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
        y = B.bsfp8_gemm_config(xt, qt, et, cfg, cps)
        y32 = B.bsfp8_gemm_config(xt, qt, et, cfg, cps, out_dtype="f32")
        torch.cuda.synchronize()
        print(_check_both(y, y32, x, G, N, K, q, e), flush=True)


@pytest.mark.parametrize("kind", ["tiny", "large"])
@pytest.mark.parametrize("M", [1, 6, 16, 64, 128, 192])
def test_extreme_exponent_bytes_built_in_plans(kind, M):
    """The plans bsfp8_gemm picks, and an explicit split, on the wo_a layout with extreme blocks."""
    G, N, K = 2, 512, 4096
    x, q, e, _ = _edge_inputs(9700 + M + (0 if kind == "tiny" else 50), M, G, N, K, kind)
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    for split in (0, 4):
        print(f"{kind} M={M} split {split} plan {B.bsfp8_plan_info(M, G, N, K, split)}", flush=True)
        y = B.bsfp8_gemm(xt, qt, et, split_k=split)
        y32 = B.bsfp8_gemm(xt, qt, et, split_k=split, out_dtype="f32")
        torch.cuda.synchronize()
        print(_check_both(y, y32, x, G, N, K, q, e), flush=True)


def test_inf_weights_nan_codes_and_exponent_byte_255():
    """A weight whose rebuilt value overflows bf16 is +-inf: its row's outputs are +-inf with the
    sign of the product (or NaN where two infinite products of opposite signs meet), as in the
    oracle's float64 sum. Exponent byte 255 turns all outputs of its 32 weight rows into NaN, and
    an e4m3 NaN code the outputs of its weight row. Every other output meets the parity rule."""
    M, G, N, K = 6, 2, 128, 512
    r = S.rng(9900)
    x = S.bf16_normal(r, (M, G * K), scale=2.0 ** -40)
    q = S.e4m3_codes(r, (G, N, K))
    e = S.exponent_bytes(r, (G, N // 32, K // 32), 110, 130)
    # (a) group 0, rows 0..31: one block at byte 254 whose codes keep the weights finite, except
    # one code of row 3 and two codes of row 7 (opposite signs of x * w -> NaN unless the signs
    # agree), which rebuild to +-inf
    e[0, 0, 5] = 254
    q[0, 0:32, 160:192] = S.cap_code_exponent_field(q[0, 0:32, 160:192], 7)
    q[0, 3, 170] = 0x7E                             # 448 * 2^127: +inf
    q[0, 7, 161] = 0x78                             # 256 * 2^127: +inf
    q[0, 7, 190] = 0xF0                             # -2^127 * 2^8: -inf
    xt, qt, et = to_gpu_bf16(x), to_gpu_u8(q), to_gpu_u8(e)
    exact = oracle.gemm_exact_f64(x, G, N, K, q, e)
    y = bf16_bits(B.bsfp8_gemm(xt, qt, et)).reshape(M, G, N)
    yv = oracle.bf16_bits_to_f64(y)
    nonfinite = ~np.isfinite(exact)
    assert nonfinite[:, 0, 3].all() and nonfinite[:, 0, 7].all() and nonfinite.sum() == 2 * M
    assert np.array_equal(np.isnan(yv), np.isnan(exact))
    inf = np.isinf(exact)
    assert np.array_equal(yv[inf], exact[inf])
    check_bf16_exact(y[~nonfinite], exact[~nonfinite], lambda: oracle.abs_products_sum(x, G, N, K, q, e)[~nonfinite],
                     K)
    # (b) exponent byte 255 on group 1, block row 2 (rows 64..95); a NaN code in group 0, row 40
    e2 = e.copy()
    q2 = q.copy()
    e2[1, 2, 9] = 255
    q2[0, 40, 300] = 0x7F
    q2[0, 41, 301] = 0xFF
    y2 = bf16_bits(B.bsfp8_gemm(xt, to_gpu_u8(q2), to_gpu_u8(e2))).reshape(M, G, N)
    y2v = oracle.bf16_bits_to_f64(y2)
    nan_rows = np.zeros((G, N), dtype=bool)
    nan_rows[1, 64:96] = True
    nan_rows[0, 40] = nan_rows[0, 41] = True
    assert np.isnan(y2v[:, nan_rows]).all()
    # elsewhere the outputs are those of the weight without the NaN entries
    keep = ~nan_rows[None].repeat(M, axis=0) & ~nonfinite
    assert np.array_equal(y2[keep], y[keep])


def test_subnormal_twin_block_through_the_gemm():
    """make_twin on a weight with an all-zero block, a block of exact e4m3 * 2^-127 values (bf16
    subnormals, accepted with exponent byte 0), blocks rebuilt from codes at exponent bytes 1..3,
    and a block of arbitrary subnormals and smallest normals (rejected, still encoded), then the
    GEMM on that twin at several row counts: codes, bytes and the ok mask equal the oracle's, and
    the output meets the parity rule."""
    G, R, D = 1, 64, 256
    r = S.rng(9950)
    q = S.e4m3_codes(r, (G, R, D))
    e = S.exponent_bytes(r, (G, R // 32, D // 32), 115, 123)
    q[0, 0:32, 32:64] = S.cap_code_exponent_field(q[0, 0:32, 32:64], 7)   # values below 2 ...
    e[0, 0, 1] = 0                                                       # ... times 2^-127
    e[0, 1, 3], e[0, 1, 4], e[0, 1, 5] = 1, 2, 3
    w = oracle.dequant_bf16(q, e)
    w[0, 0:32, 0:32] = 0                                                 # zero block
    sub = (r.integers(1, 0x80, size=(32, 32)) | (r.integers(0, 2, size=(32, 32)) << 15)).astype(np.uint16)
    sub[::3, ::5] = (0x0080 + r.integers(0, 0x80, size=sub[::3, ::5].shape)).astype(np.uint16)
    w[0, 32:64, 64:96] = sub                                             # subnormals and small normals
    ref = oracle.make_twin(w)
    t = B.bsfp8_make_twin(to_gpu_bf16(w))
    assert np.array_equal(t.q.cpu().numpy(), ref.q) and np.array_equal(t.e.cpu().numpy(), ref.e)
    assert np.array_equal(t.ok.cpu().numpy(), ref.ok)
    assert ref.e[0, 0, 0] == 0 and ref.e[0, 0, 1] == 0 and ref.e[0, 1, 2] == 0
    assert ref.ok[0, 0, 0] and ref.ok[0, 0, 1] and not ref.ok[0, 1, 2]
    print(f"subnormal twin: ok blocks {int(ref.ok.sum())}/{ref.ok.size}, bytes {ref.e[0].tolist()}", flush=True)
    for M in (1, 6, 16, 40):
        x = S.bf16_normal(S.rng(9960 + M), (M, G * D))
        y = B.bsfp8_gemm(to_gpu_bf16(x), t.q, t.e)
        torch.cuda.synchronize()
        print(M, check_bf16(bf16_bits(y), x, G, R, D, ref.q, ref.e), flush=True)


@pytest.fixture(scope="module")
def wo_a_weight():
    d = S.wo_a(2000, 1)
    W = oracle.dequant_values(d["q"], d["e"])
    return d, W, to_gpu_u8(d["q"]), to_gpu_u8(d["e"])


@pytest.mark.parametrize("M,split", [(2, 8), (4, 8), (6, 8), (8, 8), (16, 4), (32, 2)])
def test_wo_a_full_size_at_the_configurations_splits(wo_a_weight, M, split):
    """wo_a at G = 2 with the split of K the workload names (fp32 partials summed in a fixed
    order), every output against the oracle; and bitwise the same on a second call."""
    d, W, qt, et = wo_a_weight
    x = S.bf16_normal(S.rng(2200 + M), (M, 2 * 4096))
    xt = to_gpu_bf16(x)
    plan = B.bsfp8_plan_info(M, 2, 1024, 4096, split)
    print(f"wo_a M={M} split {split} plan {plan}", flush=True)
    assert plan["splits"] == split
    ws = B.workspace(M, 2, 1024, 4096, split)
    y = B.bsfp8_gemm(xt, qt, et, split_k=split, ws=ws)
    y2 = B.bsfp8_gemm(xt, qt, et, split_k=split, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    X = oracle.bf16_bits_to_f64(x).reshape(M, 2, 4096)
    exact = np.stack([X[:, g] @ W[g].T for g in range(2)], axis=1)
    print(check_bf16(bf16_bits(y), x, 2, 1024, 4096, d["q"], d["e"], exact=exact, splits=split), flush=True)
