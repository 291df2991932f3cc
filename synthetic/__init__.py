"""Seeded synthetic inputs for the block-scaled fp8 small-M GEMM workloads.

This module holds random-number generation only (NumPy PCG64, seeded): no step of the method's
arithmetic (no decode, dequantisation, encoding or contraction). Both the CPU oracle's tests and
the GPU path's tests and benchmark draw their inputs from here, as raw bit patterns:

  * activations: bf16 bit patterns of N(0,1) draws (fp32 draw, then bf16 round-half-to-even
    on the bit pattern, a generic way to make bf16 test data);
  * weights: e4m3 codes drawn uniformly over the 254 finite codes (0x7F and 0xFF, the NaNs,
    excluded; both zeros included);
  * exponent bytes: uniform integers in a stated inclusive range;
  * fp32 block scales: exact powers of two built from their exponent field.

Workload shapes follow the pages' configurations (decode/verify activations against the wo_a
weight, the shared-expert down_proj, the draft LM head). Seed = 1000 * workload id + copy index.
"""
import numpy as np

FINITE_E4M3_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_normal(r, shape, scale=1.0):
    """bf16 bit patterns (uint16) of N(0, scale^2) fp32 draws, rounded half-to-even."""
    f = (r.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_normal(r, shape, scale=1.0):
    """fp32 N(0, scale^2) draws (float32 array)."""
    return (r.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def e4m3_codes(r, shape):
    """Uniform over the finite e4m3 codes."""
    return FINITE_E4M3_CODES[r.integers(0, FINITE_E4M3_CODES.size, size=shape)]


def exponent_bytes(r, shape, lo, hi):
    """Uniform integer exponent bytes in [lo, hi]."""
    return r.integers(lo, hi + 1, size=shape).astype(np.uint8)


def pow2_scales_f32(r, shape, elo, ehi):
    """fp32 scales 2^u with u uniform in [elo, ehi] (built from the exponent field)."""
    u = r.integers(elo, ehi + 1, size=shape).astype(np.int64)
    return ((u + 127).astype(np.uint32) << 23).view(np.float32)


def small_int_bf16(r, shape, lo=-4, hi=4):
    """bf16 bit patterns of small integers (exact in bf16), for exactly-summable inputs."""
    v = r.integers(lo, hi + 1, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def perturb_one_element(w_bits, r, frac, block=32):
    """Pick `frac` of the block x block tiles of w_bits [G,R,D] and add 1 to the bit pattern of
    one nonzero element in each (one bf16 ulp away from zero). Returns (perturbed copy, mask of
    the perturbed tiles [G,R/block,D/block]). Tiles with no nonzero element are left alone."""
    w = np.array(w_bits, dtype=np.uint16, copy=True)
    G, R, D = w.shape
    rb, cb = R // block, D // block
    pick = r.random((G, rb, cb)) < frac
    mask = np.zeros((G, rb, cb), dtype=bool)
    tiles = w.reshape(G, rb, block, cb, block)
    for g, i, j in zip(*np.nonzero(pick)):
        t = tiles[g, i, :, j, :]
        nz = np.argwhere((t & 0x7FFF) != 0)
        if nz.size == 0:
            continue
        a, b = nz[r.integers(0, len(nz))]
        t[a, b] = t[a, b] + 1
        mask[g, i, j] = True
    return w, mask


# --------------------------------------------------------------------------------------------
# workloads (shapes from the pages; values synthetic)
# --------------------------------------------------------------------------------------------
def shared_down(seed, M=6, N=5120, K=576):
    """Shared-expert down_proj at TP4: X [M,K], W codes [N,K], fp32 scales [N/32,K/32] with
    exponents 2^-10..2^-4."""
    r = rng(seed)
    return dict(x=bf16_normal(r, (M, K)), q=e4m3_codes(r, (1, N, K)),
                scales=pow2_scales_f32(r, (N // 32, K // 32), -10, -4), M=M, G=1, N=N, K=K)


def wo_a(seed, M, G=2, N=1024, K=4096, elo=115, ehi=125):
    """wo_a shard: X [M, G*K], W codes [G,N,K], exponent bytes [G,N/32,K/32] in [elo, ehi]."""
    r = rng(seed)
    return dict(x=bf16_normal(r, (M, G * K)), q=e4m3_codes(r, (G, N, K)),
                e=exponent_bytes(r, (G, N // 32, K // 32), elo, ehi), M=M, G=G, N=N, K=K)


def twin_source(seed, G=4, R=1024, D=4096, elo=-12, ehi=-4):
    """Codes and block exponents e in [elo, ehi] from which an exactly-twinnable bf16 weight is
    rebuilt (by whoever consumes them: the oracle in tests, the library on the GPU)."""
    r = rng(seed)
    return dict(q=e4m3_codes(r, (G, R, D)),
                e=exponent_bytes(r, (G, R // 32, D // 32), elo + 127, ehi + 127), G=G, R=R, D=D)


def lm_head(seed, M, N=32768, K=5120, elo=118, ehi=122):
    """Draft LM head: X [M,K], W codes [1,N,K], exponent bytes 2^-9..2^-5."""
    r = rng(seed)
    return dict(x=bf16_normal(r, (M, K)), q=e4m3_codes(r, (1, N, K)),
                e=exponent_bytes(r, (1, N // 32, K // 32), elo, ehi), M=M, G=1, N=N, K=K)


# --------------------------------------------------------------------------------------------
# edge inputs: exponent bytes at the ends of the range
# --------------------------------------------------------------------------------------------
TINY_BYTES = np.array([0, 1, 2, 3], dtype=np.uint8)          # factors 2^-127 .. 2^-124
LARGE_BYTES = np.array([246, 250, 254], dtype=np.uint8)      # factors 2^119, 2^123, 2^127


def edge_exponent_bytes(r, G, N, K, extreme, lo=110, hi=130):
    """Exponent bytes [G, N/32, K/32] where block rows (32 weight rows) take one of three classes
    in turn: every block from `extreme` (an array of bytes), blocks drawn half from `extreme` and
    half from [lo, hi], and every block from [lo, hi]. Returns (bytes, class per block row)."""
    nb, kb = N // 32, K // 32
    cls = np.arange(G * nb).reshape(G, nb) % 3
    pick_ext = extreme[r.integers(0, extreme.size, size=(G, nb, kb))]
    pick_mid = r.integers(lo, hi + 1, size=(G, nb, kb)).astype(np.uint8)
    half = r.random((G, nb, kb)) < 0.5
    e = np.where(cls[:, :, None] == 0, pick_ext, np.where(cls[:, :, None] == 1, np.where(half, pick_ext, pick_mid),
                                                          pick_mid))
    return e.astype(np.uint8), cls


def cap_code_exponent_field(codes, field_max):
    """e4m3 codes with the 4-bit exponent field lowered to at most field_max (sign and fraction
    bits kept): bit-pattern surgery on the inputs, so that large block factors keep the rebuilt
    weights finite. field_max is an array broadcast against codes."""
    c = np.asarray(codes, dtype=np.uint8)
    field = (c >> 3) & 0xF
    capped = np.minimum(field, np.asarray(field_max, dtype=np.uint8))
    return ((c & 0x87) | (capped << 3)).astype(np.uint8)
