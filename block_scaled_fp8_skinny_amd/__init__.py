"""Python binding of libbsfp8 (the block-scaled fp8 small-M GEMM for MI355X).

Argument marshalling only: every function here checks tensor dtypes/devices, takes pointers,
strides and torch's current HIP stream, and calls the C entry point of the same name. All
computation runs in the HIP kernels of the library. If libbsfp8.so is missing, every call raises
(build it with `python -m block_scaled_fp8_skinny_amd.build`); there is no fallback.

Conventions (see include/bsfp8.h): bf16 tensors are torch.bfloat16; e4m3 codes are uint8 tensors
(torch.float8_e4m3fn tensors are accepted and viewed as uint8); exponent bytes are uint8.
"""
import ctypes
import os
from collections import namedtuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsfp8.so")

OK, NOT_EXACT = 0, 1
EINVAL, ESHAPE, ESCALE, ESTRIDE, EWORKSPACE, EHIP = -1, -2, -3, -4, -5, -6
OUT_BF16, OUT_F32 = 0, 1
SUM_ASCENDING, SUM_PAIRWISE = 0, 1

# name -> (restype, argtypes)
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_GEMM_ARGS = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _P, _SZ, _P, _I, _P]
_SIGS = {
    "bsfp8_strerror": (ctypes.c_char_p, [_I]),
    "bsfp8_abi_version": (_I, []),
    "bsfp8_scales_from_f32": (_I, [_P, _I64, _I64, _P, ctypes.POINTER(_I64), _P]),
    "bsfp8_make_twin": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, ctypes.POINTER(_I64), _P]),
    "bsfp8_make_twin_async": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "bsfp8_pad_k_weight": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "bsfp8_pad_k_input": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "bsfp8_dequant": (_I, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "bsfp8_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I]),
    "bsfp8_gemm_small": (_I, _GEMM_ARGS),
    "bsfp8_gemm_mid": (_I, _GEMM_ARGS),
    "bsfp8_gemm": (_I, _GEMM_ARGS),
    "bsfp8_gemm_no_alloc": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _P, _I, _P]),
    "bsfp8_num_configs": (_I, []),
    "bsfp8_read_floor": (_I, [_P, _SZ, _I, _P, _SZ, _I, _I, _P, _P, _SZ, _P]),
    "bsfp8_config_info": (_I, [_I, ctypes.POINTER(_I)]),
    "bsfp8_plan_info": (_I, [_I64, _I64, _I64, _I64, _I, _I, ctypes.POINTER(_I)]),
    "bsfp8_workspace_bytes_config": (_SZ, [_I64, _I64, _I64, _I64, _I, _I]),
    "bsfp8_gemm_config": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _I, _P, _SZ, _P, _I, _P]),
    "bsfp8_make_twin_row32": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, ctypes.POINTER(_I64), _P]),
    "bsfp8_workspace_bytes_row32": (_SZ, [_I64, _I64, _I64, _I64, _I]),
    "bsfp8_gemm_row32": (_I, _GEMM_ARGS),
    "bsfp8_gemm_row32_config": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _I, _P, _SZ, _P, _I, _P]),
    "bsfp8_quantize_mx": (_I, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "bsfp8_gemm_mx": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _I, _P]),
    "bsfp8_mx_num_configs": (_I, []),
    "bsfp8_mx_config_info": (_I, [_I, ctypes.POINTER(_I)]),
    "bsfp8_mx_plan": (_I, [_I64, _I64, _I64]),
    "bsfp8_gemm_mx_config": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _P, _I, _P]),
    "bsfp8_reduce_quantize_mx": (_I, [_P, _I64, _I64, _I64, _I, _P, _P, _P]),
    "bsfp8_workspace_bytes_mxfp8": (_SZ, [_I64, _I64, _I64, _I64, _I]),
    "bsfp8_gemm_mxfp8": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _P, _SZ, _P, _P, _P]),
    "bsfp8_workspace_bytes_mxfp8_config": (_SZ, [_I64, _I64, _I64, _I64, _I, _I]),
    "bsfp8_gemm_mxfp8_config": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I, _I, _P, _SZ, _P, _P, _P]),
}

_lib = None


class BsfpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def lib():
    """The loaded libbsfp8.so (raises when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_scaled_fp8_skinny_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


def strerror(status):
    return lib().bsfp8_strerror(int(status)).decode()


def _check(status, where):
    if status < 0:
        raise BsfpError(status, where)
    return status


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _codes(q):
    if q.dtype == torch.float8_e4m3fn:
        q = q.view(torch.uint8)
    if q.dtype != torch.uint8:
        raise TypeError("e4m3 codes must be uint8 or float8_e4m3fn")
    return q


def _need(t, dtype, name, cuda=True, numel=None, device=None):
    """Type, placement and size checks of a tensor handed to the library. The library addresses
    every buffer by the sizes it is given, so a buffer smaller than those sizes, or one on another
    device, is refused here rather than read or written out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _out_dtype(out_dtype):
    return OUT_F32 if out_dtype in ("f32", torch.float32, OUT_F32) else OUT_BF16


def _operands(x, q, e, e_numel):
    """Checked GEMM operands -> (x, M, ldx, q, G, N, K): q [G, N, K] codes, e exponent bytes of at
    least e_numel(G, N, K) elements, x [M, >= G*K] (or [M, G, K]) on q's device."""
    q = _codes(q)
    if q.dim() != 3:
        raise ValueError("q must be [G, N, K]")
    _need(q, torch.uint8, "q")
    G, N, K = q.shape
    _need(e, torch.uint8, "e", numel=e_numel(G, N, K), device=q.device)
    x, M, ldx = _x_view(x)
    if x.device != q.device:
        raise ValueError(f"x is on {x.device}, q on {q.device}")
    cols = x.shape[1] * x.shape[2] if x.dim() == 3 else x.shape[1]
    if cols < G * K:
        raise ValueError(f"x has {cols} columns per row, needs G*K = {G * K}")
    return x, M, ldx, q, G, N, K


def _block_exps(G, N, K):
    return G * (N // 32) * (K // 32)


def _row_exps(G, N, K):
    return G * N * (K // 32)


def _out(out, M, G, N, od, device):
    dtype = torch.float32 if od == OUT_F32 else torch.bfloat16
    if out is None:
        return torch.empty((M, G, N), dtype=dtype, device=device)
    _need(out, dtype, "out", numel=M * G * N, device=device)
    return out


def _ws(ws, n, device):
    """The caller's workspace (checked to hold n bytes) or a zero-filled one of n bytes."""
    if ws is None:
        return torch.zeros(n, dtype=torch.uint8, device=device) if n else None
    _need(ws, torch.uint8, "ws", numel=n, device=device)
    return ws


# ------------------------------------------------------------------------------------------------
# prepare
# ------------------------------------------------------------------------------------------------
def bsfp8_scales_from_f32(scales, exp_out=None):
    """fp32 block scales [rows, cols] -> uint8 exponent bytes. Raises BsfpError(ESCALE) when any
    scale is not a positive finite power of two (the error carries .n_bad)."""
    _need(scales, torch.float32, "scales")
    if scales.dim() != 2:
        raise ValueError("scales must be [rows, cols]")
    rows, cols = scales.shape
    if exp_out is None:
        exp_out = torch.empty((rows, cols), dtype=torch.uint8, device=scales.device)
    _need(exp_out, torch.uint8, "exp_out", numel=rows * cols, device=scales.device)
    bad = _I64(0)
    st = lib().bsfp8_scales_from_f32(_ptr(scales), rows, cols, _ptr(exp_out), ctypes.byref(bad), _stream(scales))
    if st < 0:
        err = BsfpError(st, "bsfp8_scales_from_f32")
        err.n_bad = bad.value
        raise err
    return exp_out


Twin = namedtuple("Twin", "accepted q e ok n_bad")


def bsfp8_make_twin(w):
    """bf16 weight [G, R, D] -> Twin(accepted, q [G,R,D] uint8, e [G,R/32,D/32] uint8,
    ok [G,R/32,D/32] uint8, n_bad)."""
    _need(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [G, R, D]")
    G, R, D = w.shape
    q = torch.empty((G, R, D), dtype=torch.uint8, device=w.device)
    e = torch.empty((G, R // 32, D // 32), dtype=torch.uint8, device=w.device)
    ok = torch.empty((G, R // 32, D // 32), dtype=torch.uint8, device=w.device)
    bad = _I64(0)
    st = _check(lib().bsfp8_make_twin(_ptr(w), G, R, D, _ptr(q), _ptr(e), _ptr(ok), ctypes.byref(bad),
                                      _stream(w)), "bsfp8_make_twin")
    return Twin(st == OK, q, e, ok, bad.value)


def bsfp8_make_twin_async(w, n_bad, q=None, e=None, ok=None):
    """Enqueue the encoder of bf16 w [G, R, D] without waiting: returns (q, e, ok) and adds the
    number of inexact blocks to n_bad, an int64 GPU tensor of one element that the caller zeroes
    (the twin is exact iff the count it received is 0). q, e, ok: optional outputs of the shapes
    bsfp8_make_twin returns (ok may be skipped with ok=False)."""
    _need(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [G, R, D]")
    G, R, D = w.shape
    _need(n_bad, torch.int64, "n_bad", numel=1, device=w.device)
    if q is None:
        q = torch.empty((G, R, D), dtype=torch.uint8, device=w.device)
    _need(q, torch.uint8, "q", numel=G * R * D, device=w.device)
    if e is None:
        e = torch.empty((G, R // 32, D // 32), dtype=torch.uint8, device=w.device)
    _need(e, torch.uint8, "e", numel=G * (R // 32) * (D // 32), device=w.device)
    if ok is None:
        ok = torch.empty((G, R // 32, D // 32), dtype=torch.uint8, device=w.device)
    elif ok is False:
        ok = None
    else:
        _need(ok, torch.uint8, "ok", numel=G * (R // 32) * (D // 32), device=w.device)
    _check(lib().bsfp8_make_twin_async(_ptr(w), G, R, D, _ptr(q), _ptr(e), _ptr(ok), _ptr(n_bad), _stream(w)),
           "bsfp8_make_twin_async")
    return q, e, ok


def make_twin(w):
    """(q, e) when the twin rebuilds w bit for bit, else None (the page's make_twin contract)."""
    t = bsfp8_make_twin(w)
    return (t.q, t.e) if t.accepted else None


def bsfp8_pad_k_weight(q, e, K_pad):
    """Twin codes [G,N,K] and exponents [G,N/32,K/32] -> padded to K_pad (zero codes, byte 127)."""
    q = _codes(q)
    if q.dim() != 3:
        raise ValueError("q must be [G, N, K]")
    _need(q, torch.uint8, "q")
    G, N, K = q.shape
    _need(e, torch.uint8, "e", numel=_block_exps(G, N, K), device=q.device)
    qp = torch.empty((G, N, K_pad), dtype=torch.uint8, device=q.device)
    ep = torch.empty((G, N // 32, K_pad // 32), dtype=torch.uint8, device=q.device)
    _check(lib().bsfp8_pad_k_weight(_ptr(q), _ptr(e), G, N, K, K_pad, _ptr(qp), _ptr(ep), _stream(q)),
           "bsfp8_pad_k_weight")
    return qp, ep


def _x_view(x):
    """Activation tensor -> (x, M, ldx). Accepts [M, L] with unit column stride or the page's
    [M, G, K] layout with strides (ldx, K, 1)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("x must be a bf16 GPU tensor")
    if x.dim() == 3:
        M, G, K = x.shape
        if x.stride(2) != 1 or x.stride(1) != K:
            raise ValueError("x [M, G, K] must have strides (ldx, K, 1)")
        return x, M, x.stride(0) if M > 1 else G * K
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [M, L] with unit column stride")
    return x, x.shape[0], x.stride(0) if x.shape[0] > 1 else x.shape[1]


def bsfp8_pad_k_input(x, G, K, K_pad, out=None):
    """x [M, >=G*K] (group g at columns g*K) -> [M, G*K_pad] with zero tails."""
    x, M, ldx = _x_view(x)
    cols = x.shape[1] * x.shape[2] if x.dim() == 3 else x.shape[1]
    if cols < G * K:
        raise ValueError(f"x has {cols} columns per row, needs G*K = {G * K}")
    if out is None:
        out = torch.empty((M, G * K_pad), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", numel=M * G * K_pad, device=x.device)
    _check(lib().bsfp8_pad_k_input(_ptr(x), ldx, M, G, K, K_pad, _ptr(out), _stream(x)), "bsfp8_pad_k_input")
    return out


def bsfp8_dequant(q, e, out=None):
    """Twin -> bf16 weight [G, N, K], exact."""
    q = _codes(q)
    if q.dim() != 3:
        raise ValueError("q must be [G, N, K]")
    _need(q, torch.uint8, "q")
    G, N, K = q.shape
    _need(e, torch.uint8, "e", numel=_block_exps(G, N, K), device=q.device)
    if out is None:
        out = torch.empty((G, N, K), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", numel=G * N * K, device=q.device)
    _check(lib().bsfp8_dequant(_ptr(q), _ptr(e), G, N, K, _ptr(out), _stream(q)), "bsfp8_dequant")
    return out


# ------------------------------------------------------------------------------------------------
# per call
# ------------------------------------------------------------------------------------------------
def bsfp8_workspace_bytes(M, G, N, K, split_k=0):
    return int(lib().bsfp8_workspace_bytes(M, G, N, K, split_k))


def workspace(M, G, N, K, split_k=0, device="cuda"):
    """A zero-filled workspace tensor for these sizes (or None when none is needed)."""
    n = bsfp8_workspace_bytes(M, G, N, K, split_k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _gemm(entry, x, q, e, split_k, ws, out, out_dtype):
    x, M, ldx, q, G, N, K = _operands(x, q, e, _block_exps)
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, x.device)
    ws = _ws(ws, bsfp8_workspace_bytes(max(M, 1), G, N, K, split_k), x.device)
    wsb = ws.numel() if ws is not None else 0
    fn = getattr(lib(), entry)
    _check(fn(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), split_k, _ptr(ws), wsb, _ptr(out), od, _stream(x)), entry)
    return out


def bsfp8_gemm(x, q, e, split_k=0, ws=None, out=None, out_dtype="bf16"):
    """Y [M, G, N] = per group X[:, g*K:(g+1)*K] @ W_g^T, W_g rebuilt from the twin (q, e)."""
    return _gemm("bsfp8_gemm", x, q, e, split_k, ws, out, out_dtype)


NO_ALLOC_SCRATCH_BYTES = 16 << 20   # BSFP8_NO_ALLOC_SCRATCH_BYTES of include/bsfp8.h


def bsfp8_gemm_no_alloc(x, q, e, split_k=0, out=None, out_dtype="bf16"):
    """bsfp8_gemm without a workspace: a split plan uses the library's static per-GPU scratch
    (calls that can overlap on one GPU must not be made)."""
    x, M, ldx, q, G, N, K = _operands(x, q, e, _block_exps)
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, x.device)
    _check(lib().bsfp8_gemm_no_alloc(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), split_k, _ptr(out), od,
                                     _stream(x)), "bsfp8_gemm_no_alloc")
    return out


def bsfp8_gemm_small(x, q, e, split_k=0, ws=None, out=None, out_dtype="bf16"):
    return _gemm("bsfp8_gemm_small", x, q, e, split_k, ws, out, out_dtype)


def bsfp8_gemm_mid(x, q, e, split_k=0, ws=None, out=None, out_dtype="bf16"):
    return _gemm("bsfp8_gemm_mid", x, q, e, split_k, ws, out, out_dtype)


# ------------------------------------------------------------------------------------------------
# tuning interface (include/bsfp8_tuning.h)
# ------------------------------------------------------------------------------------------------
def bsfp8_num_configs():
    return int(lib().bsfp8_num_configs())


def bsfp8_read_floor(t, nbytes=None, nwg=256, sink=None, out=None, slab=None, slab_groups=1, interleave=False):
    """Plain-read floor: one kernel that reads the first nbytes (default: all) of the GPU tensor t
    once with the GEMM's load shape and computes nothing else (a measurement aid; nbytes = 0 is a
    bare launch). sink: uint32 [nwg] on t's device (allocated when None). slab: a contiguous GPU
    tensor of slab_groups equal parts; every workgroup also reads the part of its group whole
    (the activation rows every workgroup of a GEMM reads), before its share of t, or spread over
    the steps of that share with interleave=True; or None. out: a contiguous GPU tensor of a
    multiple of 16 bytes that the kernel also writes whole (the read + write floor of a GEMM
    storing that many output bytes), or None. Returns the sink."""
    nb = t.numel() * t.element_size() if nbytes is None else int(nbytes)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("t must be a contiguous GPU tensor")
    if nb > t.numel() * t.element_size():
        raise ValueError(f"t holds {t.numel() * t.element_size()} bytes, {nb} requested")
    if sink is None:
        sink = torch.empty(nwg, dtype=torch.int32, device=t.device)
    _need(sink, torch.int32, "sink", numel=nwg, device=t.device)
    ob = 0
    if out is not None:
        if not out.is_cuda or not out.is_contiguous() or out.device != t.device:
            raise ValueError("out must be a contiguous GPU tensor on t's device")
        ob = out.numel() * out.element_size()
    sb = 0
    if slab is not None:
        if not slab.is_cuda or not slab.is_contiguous() or slab.device != t.device:
            raise ValueError("slab must be a contiguous GPU tensor on t's device")
        total = slab.numel() * slab.element_size()
        if slab_groups < 1 or total % slab_groups:
            raise ValueError(f"slab of {total} bytes does not split into {slab_groups} groups")
        sb = total // slab_groups
    _check(lib().bsfp8_read_floor(_ptr(t), nb, nwg, _ptr(slab), sb, int(slab_groups), 1 if interleave else 0,
                                  _ptr(sink), _ptr(out), ob, _stream(t)), "bsfp8_read_floor")
    return sink


def bsfp8_config_info(cfg):
    out = (_I * 8)()
    _check(lib().bsfp8_config_info(cfg, out), "bsfp8_config_info")
    return dict(BM=out[0], NB=out[1], threads=out[2], CW=out[3], NWN=out[4], NWK=out[5], direct=out[6] in (1, 2, 4),
                kind=out[6], row_scales=out[7] & 1, xcds_per_group=out[7] >> 8)


def bsfp8_plan_info(M, G, N, K, split_k=0, path=2):
    out = (_I * 8)()
    _check(lib().bsfp8_plan_info(M, G, N, K, split_k, path, out), "bsfp8_plan_info")
    keys = ("cfg", "BM", "NB", "kchunks", "cps", "splits", "mblocks", "workgroups")
    return dict(zip(keys, list(out)))


def bsfp8_workspace_bytes_config(M, G, N, K, cfg, cps):
    return int(lib().bsfp8_workspace_bytes_config(M, G, N, K, cfg, cps))


def bsfp8_gemm_config(x, q, e, cfg, cps, ws=None, out=None, out_dtype="bf16"):
    x, M, ldx, q, G, N, K = _operands(x, q, e, _block_exps)
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, x.device)
    ws = _ws(ws, bsfp8_workspace_bytes_config(max(M, 1), G, N, K, cfg, cps), x.device)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().bsfp8_gemm_config(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), cfg, cps, _ptr(ws), wsb,
                                   _ptr(out), od, _stream(x)), "bsfp8_gemm_config")
    return out


# ------------------------------------------------------------------------------------------------
# MXFP8 activations and the fp8 x fp8 GEMM
# ------------------------------------------------------------------------------------------------
def bsfp8_quantize_mx(x, L=None, xq=None, xs=None):
    """bf16 activations [M, >= L] -> (codes uint8 [M, L], scale bytes uint8 [M, L/32])."""
    x, M, ldx = _x_view(x)
    if x.dim() == 3:
        raise ValueError("x must be [M, L]")
    L = x.shape[1] if L is None else L
    if L > x.shape[1]:
        raise ValueError(f"L = {L} exceeds the {x.shape[1]} columns of x")
    if xq is None:
        xq = torch.empty((M, L), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((M, L // 32), dtype=torch.uint8, device=x.device)
    _need(xq, torch.uint8, "xq", numel=M * L, device=x.device)
    _need(xs, torch.uint8, "xs", numel=M * (L // 32), device=x.device)
    _check(lib().bsfp8_quantize_mx(_ptr(x), ldx, M, L, _ptr(xq), _ptr(xs), _stream(x)), "bsfp8_quantize_mx")
    return xq, xs


def _mx_args(xq, xs, q, e, out, out_dtype):
    q = _codes(q)
    if q.dim() != 3:
        raise ValueError("q must be [G, N, K]")
    _need(q, torch.uint8, "q")
    G, N, K = q.shape
    _need(e, torch.uint8, "e", numel=_block_exps(G, N, K), device=q.device)
    xq = _codes(xq)
    if xq.dtype != torch.uint8 or xq.dim() != 2 or xq.stride(1) != 1 or not xq.is_cuda:
        raise ValueError("xq must be a uint8 GPU tensor [M, ldq] with unit column stride")
    if not isinstance(xs, torch.Tensor) or xs.dtype != torch.uint8 or xs.dim() != 2 or xs.stride(1) != 1:
        raise ValueError("xs must be a uint8 tensor [M, ldq/32] with unit column stride")
    if xq.device != q.device or xs.device != q.device:
        raise ValueError("xq, xs, q and e must be on one GPU")
    M = xq.shape[0]
    ldq = xq.stride(0) if M > 1 else xq.shape[1]
    if M > 1 and xs.stride(0) * 32 != ldq:
        raise ValueError("xs must be uint8 [M, ldq/32] with rows aligned to the codes")
    if xs.shape[0] != M or xq.shape[1] < G * K or xs.shape[1] < G * K // 32:
        raise ValueError(f"xq [M, >= G*K] and xs [M, >= G*K/32] needed (G*K = {G * K})")
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, xq.device)
    return xq, q, M, ldq, G, N, K, od, out


def bsfp8_gemm_mx(xq, xs, q, e, out=None, out_dtype="bf16"):
    """Y [M, G, N] = per group Xmx[:, g*K:(g+1)*K] @ W_g^T on the block-scaled fp8 MFMA."""
    xq, q, M, ldq, G, N, K, od, out = _mx_args(xq, xs, q, e, out, out_dtype)
    _check(lib().bsfp8_gemm_mx(_ptr(xq), _ptr(xs), ldq, M, G, N, K, _ptr(q), _ptr(e), _ptr(out), od, _stream(xq)),
           "bsfp8_gemm_mx")
    return out


def bsfp8_mx_num_configs():
    return int(lib().bsfp8_mx_num_configs())


def bsfp8_mx_config_info(cfg):
    out = (_I * 6)()
    _check(lib().bsfp8_mx_config_info(cfg, out), "bsfp8_mx_config_info")
    return dict(BM=out[0], NB=out[1], threads=out[2], SC=out[3], stages=out[4], NWK=out[5])


def bsfp8_mx_plan(M, G, N):
    return _check(int(lib().bsfp8_mx_plan(M, G, N)), "bsfp8_mx_plan")


def bsfp8_gemm_mx_config(xq, xs, q, e, cfg, out=None, out_dtype="bf16"):
    xq, q, M, ldq, G, N, K, od, out = _mx_args(xq, xs, q, e, out, out_dtype)
    _check(lib().bsfp8_gemm_mx_config(_ptr(xq), _ptr(xs), ldq, M, G, N, K, _ptr(q), _ptr(e), cfg, _ptr(out), od,
                                      _stream(xq)), "bsfp8_gemm_mx_config")
    return out


# ------------------------------------------------------------------------------------------------
# twins with one exponent per row and 32 columns
# ------------------------------------------------------------------------------------------------
def bsfp8_make_twin_row32(w):
    """bf16 weight [G, N, K] -> Twin(accepted, q [G,N,K] uint8, e [G,N,K/32] uint8,
    ok [G,N,K/32] uint8, n_bad)."""
    _need(w, torch.bfloat16, "w")
    if w.dim() != 3:
        raise ValueError("w must be [G, N, K]")
    G, N, K = w.shape
    q = torch.empty((G, N, K), dtype=torch.uint8, device=w.device)
    e = torch.empty((G, N, K // 32), dtype=torch.uint8, device=w.device)
    ok = torch.empty((G, N, K // 32), dtype=torch.uint8, device=w.device)
    bad = _I64(0)
    st = _check(lib().bsfp8_make_twin_row32(_ptr(w), G, N, K, _ptr(q), _ptr(e), _ptr(ok), ctypes.byref(bad),
                                            _stream(w)), "bsfp8_make_twin_row32")
    return Twin(st == OK, q, e, ok, bad.value)


def bsfp8_workspace_bytes_row32(M, G, N, K, split_k=0):
    return int(lib().bsfp8_workspace_bytes_row32(M, G, N, K, split_k))


def workspace_row32(M, G, N, K, split_k=0, device="cuda"):
    n = bsfp8_workspace_bytes_row32(M, G, N, K, split_k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def bsfp8_gemm_row32(x, q, e, split_k=0, ws=None, out=None, out_dtype="bf16"):
    """Y [M, G, N] = per group X[:, g*K:(g+1)*K] @ W_g^T with W rebuilt from a row-scale twin
    (e [G, N, K/32]); up to 16 rows."""
    x, M, ldx, q, G, N, K = _operands(x, q, e, _row_exps)
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, x.device)
    ws = _ws(ws, bsfp8_workspace_bytes_row32(max(M, 1), G, N, K, split_k), x.device)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().bsfp8_gemm_row32(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), split_k, _ptr(ws), wsb, _ptr(out), od,
                                  _stream(x)), "bsfp8_gemm_row32")
    return out


def bsfp8_gemm_row32_config(x, q, e, cfg, cps, ws=None, out=None, out_dtype="bf16"):
    x, M, ldx, q, G, N, K = _operands(x, q, e, _row_exps)
    od = _out_dtype(out_dtype)
    out = _out(out, M, G, N, od, x.device)
    ws = _ws(ws, bsfp8_workspace_bytes_config(max(M, 1), G, N, K, cfg, cps), x.device)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().bsfp8_gemm_row32_config(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), cfg, cps, _ptr(ws), wsb,
                                         _ptr(out), od, _stream(x)), "bsfp8_gemm_row32_config")
    return out


# ------------------------------------------------------------------------------------------------
# MXFP8 output epilogue
# ------------------------------------------------------------------------------------------------
def _mx_out(M, L, device, yq, ys):
    if yq is None:
        yq = torch.empty((M, L), dtype=torch.uint8, device=device)
    if ys is None:
        ys = torch.empty((M, L // 32), dtype=torch.uint8, device=device)
    _need(yq, torch.uint8, "yq", numel=M * L, device=device)
    _need(ys, torch.uint8, "ys", numel=M * (L // 32), device=device)
    return yq, ys


def bsfp8_reduce_quantize_mx(part, order=SUM_PAIRWISE, yq=None, ys=None):
    """fp32 partials [S, M, L] -> (codes uint8 [M, L], scale bytes uint8 [M, L/32]): the fixed-order
    fp32 sum of the S partials, quantised to MXFP8 along L."""
    _need(part, torch.float32, "part")
    if part.dim() != 3:
        raise ValueError("part must be [S, M, L]")
    S, M, L = part.shape
    yq, ys = _mx_out(M, L, part.device, yq, ys)
    _check(lib().bsfp8_reduce_quantize_mx(_ptr(part), S, M, L, int(order), _ptr(yq), _ptr(ys), _stream(part)),
           "bsfp8_reduce_quantize_mx")
    return yq, ys


def bsfp8_workspace_bytes_mxfp8(M, G, N, K, split_k=0):
    return int(lib().bsfp8_workspace_bytes_mxfp8(M, G, N, K, split_k))


def workspace_mxfp8(M, G, N, K, split_k=0, device="cuda"):
    """A workspace tensor for bsfp8_gemm_mxfp8 (its contents need no clearing)."""
    return torch.empty(bsfp8_workspace_bytes_mxfp8(M, G, N, K, split_k), dtype=torch.uint8, device=device)


def bsfp8_gemm_mxfp8(x, q, e, split_k=0, ws=None, yq=None, ys=None):
    """The GEMM of bsfp8_gemm with the MXFP8 epilogue -> (codes uint8 [M, G*N], scale bytes uint8
    [M, G*N/32])."""
    x, M, ldx, q, G, N, K = _operands(x, q, e, _block_exps)
    yq, ys = _mx_out(M, G * N, x.device, yq, ys)
    if ws is None and M > 0:
        ws = workspace_mxfp8(M, G, N, K, split_k, device=x.device)
    elif ws is not None:
        _need(ws, torch.uint8, "ws", numel=bsfp8_workspace_bytes_mxfp8(M, G, N, K, split_k), device=x.device)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().bsfp8_gemm_mxfp8(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), split_k, _ptr(ws), wsb,
                                  _ptr(yq), _ptr(ys), _stream(x)), "bsfp8_gemm_mxfp8")
    return yq, ys


def bsfp8_workspace_bytes_mxfp8_config(M, G, N, K, cfg, cps):
    return int(lib().bsfp8_workspace_bytes_mxfp8_config(M, G, N, K, cfg, cps))


def bsfp8_gemm_mxfp8_config(x, q, e, cfg, cps, ws=None, yq=None, ys=None):
    x, M, ldx, q, G, N, K = _operands(x, q, e, _block_exps)
    yq, ys = _mx_out(M, G * N, x.device, yq, ys)
    n = bsfp8_workspace_bytes_mxfp8_config(M, G, N, K, cfg, cps) if M > 0 else 0
    if ws is None and M > 0:
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    elif ws is not None:
        _need(ws, torch.uint8, "ws", numel=n, device=x.device)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().bsfp8_gemm_mxfp8_config(_ptr(x), ldx, M, G, N, K, _ptr(q), _ptr(e), cfg, cps, _ptr(ws), wsb,
                                         _ptr(yq), _ptr(ys), _stream(x)), "bsfp8_gemm_mxfp8_config")
    return yq, ys
