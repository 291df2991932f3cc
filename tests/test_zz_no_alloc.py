"""GPU checks of bsfp8_gemm_no_alloc, the GEMM entry point that allocates nothing: a plan that
needs a workspace runs on the library's static per-GPU scratch instead of a caller's buffer.

Each case makes two calls in a row on the shared array, the second with a smaller input, and
compares every output bitwise with bsfp8_gemm (same plan, same kernels, a zero-filled workspace of
its own); the smaller wo_a-shaped case is also checked against the oracle. A plan whose workspace
exceeds the array is refused before anything is enqueued.
"""
import pytest
import torch

import block_scaled_fp8_skinny_amd as B
import synthetic as S
from parity import bf16_bits, check_bf16, check_f32, to_gpu_bf16, to_gpu_u8

pytestmark = pytest.mark.gpu


def _operands(seed, M, G, N, K):
    d = S.wo_a(seed, M, G=G, N=N, K=K)
    return d, to_gpu_bf16(d["x"]), to_gpu_u8(d["q"]), to_gpu_u8(d["e"])


def _with_ws(xt, qt, et, split, out_dtype):
    M, G, N, K = xt.shape[0], qt.shape[0], qt.shape[1], qt.shape[2]
    ws = B.workspace(M, G, N, K, split)
    return B.bsfp8_gemm(xt, qt, et, split_k=split, ws=ws, out_dtype=out_dtype)


def _same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


# (first call, second smaller call): (M, G, N, K, split_k, out dtype)
CASES = [
    # one-pass kernels with the pairwise exchange slots
    ((8, 4, 1024, 4096, 8, "bf16"), (4, 2, 256, 1024, 8, "bf16")),
    ((16, 2, 1024, 4096, 4, "f32"), (3, 1, 512, 2048, 2, "f32")),
    # mid row counts: register kernel, then slab kernel, both with exchange slots
    ((128, 2, 1024, 4096, 4, "bf16"), (64, 1, 512, 2048, 2, "bf16")),
    # plans without a workspace
    ((6, 4, 1024, 4096, 0, "bf16"), (2, 1, 256, 512, 0, "f32")),
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: "M%d_G%d_N%d_K%d_s%d_%s" % c)
def test_no_alloc_matches_gemm_on_two_calls(first, second):
    outs = []
    for i, (M, G, N, K, split, od) in enumerate((first, second)):
        plan = B.bsfp8_plan_info(M, G, N, K, split)
        kind = B.bsfp8_config_info(plan["cfg"])["kind"]
        ws_bytes = B.bsfp8_workspace_bytes(M, G, N, K, split)
        print(f"no_alloc call {i}: M={M} G={G} N={N} K={K} split {split} {od} plan {plan} kind {kind} "
              f"ws {ws_bytes}", flush=True)
        assert ws_bytes <= B.NO_ALLOC_SCRATCH_BYTES
        if split > 1:
            assert plan["splits"] == split and ws_bytes > 0
        d, xt, qt, et = _operands(5100 + 17 * i + M, M, G, N, K)
        y = B.bsfp8_gemm_no_alloc(xt, qt, et, split_k=split, out_dtype=od)
        outs.append((d, xt, qt, et, split, od, y))
    for d, xt, qt, et, split, od, y in outs:
        ref = _with_ws(xt, qt, et, split, od)
        torch.cuda.synchronize()
        assert _same(y, ref)
    # the smaller call against the oracle as well
    d, xt, qt, et, split, od, y = outs[1]
    if od == "bf16":
        print(check_bf16(bf16_bits(y), d["x"], d["G"], d["N"], d["K"], d["q"], d["e"], splits=max(split, 1)),
              flush=True)
    else:
        check_f32(y.cpu().numpy(), d["x"], d["G"], d["N"], d["K"], d["q"], d["e"], splits=max(split, 1))


def test_no_alloc_repeated_split_calls_and_a_side_stream():
    """The exchange slots are cleared by each call: five split calls in a row on the default
    stream and one on another stream (default priority) all equal bsfp8_gemm."""
    M, G, N, K, split = 8, 2, 1024, 4096, 8
    d, xt, qt, et = _operands(5300, M, G, N, K)
    ref = _with_ws(xt, qt, et, split, "bf16")
    ys = [B.bsfp8_gemm_no_alloc(xt, qt, et, split_k=split) for _ in range(5)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y_side = B.bsfp8_gemm_no_alloc(xt, qt, et, split_k=split)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for y in ys + [y_side]:
        assert _same(y, ref)


def test_no_alloc_refuses_a_plan_beyond_the_scratch():
    M, G, N, K, split = 256, 1, 8192, 4096, 8
    need = B.bsfp8_workspace_bytes(M, G, N, K, split)
    print(f"workspace {need} > scratch {B.NO_ALLOC_SCRATCH_BYTES}", flush=True)
    assert need > B.NO_ALLOC_SCRATCH_BYTES
    xt = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    qt = torch.zeros((1, N, K), dtype=torch.uint8, device="cuda")
    et = torch.full((1, N // 32, K // 32), 127, dtype=torch.uint8, device="cuda")
    out = torch.full((M, 1, N), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    with pytest.raises(B.BsfpError) as err:
        B.bsfp8_gemm_no_alloc(xt, qt, et, split_k=split, out=out)
    assert err.value.status == -5          # BSFP8_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == 7).all())
