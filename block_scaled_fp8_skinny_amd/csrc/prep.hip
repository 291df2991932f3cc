// Preparation kernels of the block-scaled fp8 weight path for gfx950: scale ingestion, the
// exact-twin encoder, K padding and standalone dequantisation.

#include "device.h"

namespace bsfp8 {
namespace {

// ---------------------------------------------------------------------------------------------
// fp32 block scales -> exponent bytes (page "shared_pad_k.py", _pad_weight: positive powers of
// two only). One thread per scale; refused scales count into *bad and get byte 0.
// ---------------------------------------------------------------------------------------------
__global__ void scales_kernel(const uint32_t* s, int64_t n, uint8_t* out, unsigned long long* bad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = s[i];
  const uint32_t ef = (u >> 23) & 0xFF;
  const bool ok = (u & 0x807FFFFFu) == 0 && ef >= 1 && ef <= 254;
  out[i] = ok ? (uint8_t)ef : 0;
  if (!ok) atomicAdd(bad, 1ull);
}

// ---------------------------------------------------------------------------------------------
// Twin encoder (page "wo_a_w8.py", make_twin). One wave per block row (32 rows) and strip of 128
// columns (4 blocks): lane (r4, c16) = (lane / 16, lane % 16) holds columns 8*c16 .. 8*c16+7 of
// the strip in rows r4, r4 + 4, ..., r4 + 28. Each load then reads four rows x 256 contiguous
// bytes (HBM streams this near its best rate; a wave per block reading 64 bytes of each of 32
// rows ran at about a quarter of the peak), and block b of the strip is the 16 lanes with
// c16 / 4 == b (reductions by lane exchanges 1, 2, 16, 32).
// The codes come from the hardware's scaled conversion of bf16 pairs (v_cvt_scalef32_pk_fp8_bf16
// divides by 2^(scale exponent field - 127) and rounds to nearest even; with |w| / 2^e <= 448 by
// the choice of e it neither saturates nor overflows) and the rebuild from its inverse: both are
// exact for every bf16 value and every e in [-127, 127] (measured against the integer encoder),
// two elements per instruction.
// ---------------------------------------------------------------------------------------------
constexpr int TWIN_STRIP = 128;                     // columns per wave: 16 lanes x 8

// Least e with max(amax, 2^-126) <= 448 * 2^e, from the bf16 pattern of amax (finite):
// amax = (128 + f) * 2^(E - 134); 448 * 2^e = 7 * 2^(6 + e). For a normal amax the bound holds
// with e = E - 135 when f <= 96 (mantissa <= 1.75) and needs e = E - 134 otherwise. Zero and
// subnormal amax are raised to 2^-126, which gives e = -134, clamped to -127.
__device__ __forceinline__ int block_exp(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 7), f = (int)(amax_bits & 0x7F);
  int e = (E == 0) ? -134 : (f <= 96 ? E - 135 : E - 134);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__global__ void __launch_bounds__(256) make_twin_kernel(const uint16_t* w, int64_t D, int64_t nstrips,
                                                        int64_t nwaves, uint8_t* q, uint8_t* e,
                                                        uint8_t* okv, unsigned long long* bad) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= nwaves) return;                        // whole wave exits together
  const int r4 = lane >> 4, c16 = lane & 15;
  const int64_t strip = wid % nstrips;
  const int64_t grb = wid / nstrips;                // g * R/32 + block row
  const int64_t col = strip * TWIN_STRIP + c16 * 8;
  const bool live = col < D;                        // D % 32 == 0: the 4 lanes of a block agree
  const int64_t row0 = grb * 32 + r4;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = live ? *reinterpret_cast<const uint4*>(w + (row0 + 4 * i) * D + col) : make_uint4(0, 0, 0, 0);
  // block maximum of the magnitude patterns (inf and NaN patterns exceed every finite one)
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = d[j] & 0x7FFF, hi = (d[j] >> 16) & 0x7FFF;
      amax = max(amax, max(lo, hi));
    }
  }
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) {
    if (off == 4 || off == 8) continue;             // lanes 4b .. 4b+3 of each row group
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  }
  const bool finite = amax < 0x7F80;
  const int eb = block_exp(finite ? amax : 0);
  const float scale = __uint_as_float((uint32_t)(eb + 127) << 23);   // 2^eb (field 0: 2^-127)
  uint32_t same = 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = e4m3x2_bf16(d[j], scale);
      const uint32_t back = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], scale, false));
      same &= back == d[j] ? 1u : 0u;
    }
    uint2 out = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
    if (!finite) out = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (live) *reinterpret_cast<uint2*>(q + (row0 + 4 * i) * D + col) = out;
  }
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) {
    if (off == 4 || off == 8) continue;
    same &= (uint32_t)__shfl_xor((int)same, off);
  }
  const bool ok = same && finite;
  if (live && r4 == 0 && (c16 & 3) == 0) {
    const int64_t blk = grb * (D / 32) + col / 32;
    e[blk] = finite ? (uint8_t)(eb + 127) : (uint8_t)255;
    if (okv) okv[blk] = ok ? 1 : 0;
    if (!ok) atomicAdd(bad, 1ull);
  }
}

// ---------------------------------------------------------------------------------------------
// Twin encoder with one exponent per row and 32 columns (page "recipes/docker-images/mia-tp4/
// docs/tp4-adapters.md", row draft_main_proj: e4m3 with per-(row, 32-column) power-of-two
// scales, checked to reproduce the weight exactly). The per-block rule is the 32x32 encoder's.
// Two lanes per 1x32 block, sixteen values each; a block's 64 bytes are contiguous, so lane t
// reads values 16t .. 16t + 15 of the flat weight. Codes and rebuild by the hardware's scaled
// conversions, as in make_twin_kernel.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) make_twin_row32_kernel(const uint16_t* w, int64_t nblocks, uint8_t* q,
                                                              uint8_t* e, uint8_t* okv, unsigned long long* bad) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 1;
  const bool live = blk < nblocks;
  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
  if (live) {
    const uint4* src = reinterpret_cast<const uint4*>(w + t * 16);
    v0 = src[0];
    v1 = src[1];
  }
  const uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[2 * i] = d[i] & 0xFFFF;
    h[2 * i + 1] = d[i] >> 16;
  }
  uint32_t amax = 0, nonfinite = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = h[i] & 0x7FFF;
    nonfinite |= m >= 0x7F80 ? 1u : 0u;
    amax = m > amax ? m : amax;
  }
  // the two lanes of a block are adjacent in the wave
  const uint32_t o = (uint32_t)__shfl_xor((int)amax, 1);
  amax = o > amax ? o : amax;
  nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, 1);
  const int eb = block_exp(nonfinite ? 0u : amax);
  const uint32_t eb_byte = (uint32_t)(eb + 127);
  const float scale = __uint_as_float(eb_byte << 23);   // 2^e, for the codes and the rebuild
  // codes of each bf16 pair (w / 2^e, RNE; within +-448 by the choice of e), rebuilt and compared
  uint32_t c2[8], same = 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c2[i] = e4m3x2_bf16(d[i], scale);
    same &= bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c2[i], scale, false)) == d[i] ? 1u : 0u;
  }
  same &= (uint32_t)__shfl_xor((int)same, 1);
  const bool ok = same && !nonfinite;
  uint4 out = make_uint4(c2[0] | (c2[1] << 16), c2[2] | (c2[3] << 16), c2[4] | (c2[5] << 16), c2[6] | (c2[7] << 16));
  if (nonfinite) out = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
  if (live) {
    *reinterpret_cast<uint4*>(q + t * 16) = out;
    if ((t & 1) == 0) {
      e[blk] = nonfinite ? (uint8_t)255 : (uint8_t)eb_byte;
      if (okv) okv[blk] = ok ? 1 : 0;
      if (!ok) atomicAdd(bad, 1ull);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// K padding of a twin (page "shared_pad_k.py", _pad_weight): zero codes, unit exponents.
// One thread per 16 codes of the padded weight; one thread per padded exponent byte.
// ---------------------------------------------------------------------------------------------
__global__ void pad_codes_kernel(const uint8_t* q, int64_t rows, int64_t K, int64_t K_pad,
                                 uint8_t* q_pad) {
  const int64_t per_row = K_pad / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row, c = (i % per_row) * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (c < K) v = *reinterpret_cast<const uint4*>(q + r * K + c);
  *reinterpret_cast<uint4*>(q_pad + r * K_pad + c) = v;
}

__global__ void pad_exps_kernel(const uint8_t* e, int64_t rows, int64_t kb, int64_t kb_pad,
                                uint8_t* e_pad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * kb_pad) return;
  const int64_t r = i / kb_pad, c = i % kb_pad;
  e_pad[i] = c < kb ? e[r * kb + c] : (uint8_t)127;
}

// Activations (page "shared_pad_k.py", _pad_input): x [M][ldx] -> x_pad [M][G*K_pad] with a
// zero tail per group. Vector form: one thread per 8 values; scalar form for odd strides.
__global__ void pad_input_vec_kernel(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t K,
                                     int64_t K_pad, uint16_t* x_pad) {
  const int64_t per_row = G * K_pad / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * per_row) return;
  const int64_t m = i / per_row, c = (i % per_row) * 8;
  const int64_t g = c / K_pad, k = c % K_pad;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (k < K) v = *reinterpret_cast<const uint4*>(x + m * ldx + g * K + k);
  *reinterpret_cast<uint4*>(x_pad + m * G * K_pad + c) = v;
}

__global__ void pad_input_scalar_kernel(const uint16_t* x, int64_t ldx, int64_t M, int64_t G,
                                        int64_t K, int64_t K_pad, uint16_t* x_pad) {
  const int64_t per_row = G * K_pad;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * per_row) return;
  const int64_t m = i / per_row, c = i % per_row;
  const int64_t g = c / K_pad, k = c % K_pad;
  x_pad[i] = k < K ? x[m * ldx + g * K + k] : (uint16_t)0;
}

// ---------------------------------------------------------------------------------------------
// Standalone dequantisation (page "wo_a_w8.py", _dequant_kernel). A workgroup converts 8 x 256
// consecutive 8-code pieces of the flattened [rows][K] codes, thread t the pieces t, t + 256, ...:
// a lane loads 8 bytes and stores 16, so every wave load is 512 contiguous bytes and every wave
// store one contiguous kilobyte (16-code pieces, whose two 16-byte stores each left every other
// 16 bytes of a 2 KB span to the other store, were slower), and a thread keeps eight loads in
// flight. Indices are 32-bit (a launch covers fewer than 2^31 codes) and the row of a piece comes
// from a multiply-and-shift division. The bf16 output is written with non-temporal stores (it is
// not read again by this kernel, and streaming it past the caches took a [4, 1024, 4096] layer
// from 12.6 to 11.0 us); four pieces per thread: 10.4 us.
// ---------------------------------------------------------------------------------------------
constexpr int DQ_UNROLL = 4;

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* q, const uint8_t* e, uint32_t npieces,
                                                      uint32_t per_row, FastDiv row_of, uint32_t K, uint16_t* w) {
  const uint32_t base = blockIdx.x * (256u * DQ_UNROLL) + threadIdx.x;
  const uint32_t kb = K / 32;
  uint2 v[DQ_UNROLL];
  uint32_t b[DQ_UNROLL];
  uint32_t o[DQ_UNROLL];
#pragma unroll
  for (int u = 0; u < DQ_UNROLL; ++u) {
    const uint32_t i = base + u * 256u;
    if (i < npieces) {
      const uint32_t r = (uint32_t)fdiv((int)i, row_of), c = (i - r * per_row) * 8u;
      o[u] = r * K + c;
      // rows run over [G*N]; block rows over [G*N/32] in the same order
      b[u] = e[(r / 32) * kb + c / 32];
      v[u] = *reinterpret_cast<const uint2*>(q + o[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < DQ_UNROLL; ++u) {
    const uint32_t i = base + u * 256u;
    if (i >= npieces) continue;
    const float sc = __uint_as_float(b[u] << 23);
    const u32x4_t out = {bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[u].x, sc, false)),
                         bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[u].x, sc, true)),
                         bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[u].y, sc, false)),
                         bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[u].y, sc, true))};
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4_t*>(w + o[u]));
  }
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

int launch_scales_from_f32(const float* s, int64_t n, uint8_t* out, unsigned long long* bad,
                           hipStream_t stream) {
  if (n == 0) return BSFP8_OK;
  hipLaunchKernelGGL(scales_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(s), n, out, bad);
  return hip_status(hipGetLastError());
}

int launch_make_twin(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q, uint8_t* e,
                     uint8_t* ok, unsigned long long* bad, hipStream_t stream) {
  const int64_t nstrips = (D + TWIN_STRIP - 1) / TWIN_STRIP;
  const int64_t nwaves = G * (R / 32) * nstrips;
  if (nwaves == 0) return BSFP8_OK;
  hipLaunchKernelGGL(make_twin_kernel, dim3(grid_for(nwaves, 4)), dim3(256), 0, stream, w, D, nstrips,
                     nwaves, q, e, ok, bad);
  return hip_status(hipGetLastError());
}

int launch_make_twin_row32(const uint16_t* w, int64_t G, int64_t N, int64_t K, uint8_t* q, uint8_t* e,
                           uint8_t* ok, unsigned long long* bad, hipStream_t stream) {
  const int64_t nblocks = G * N * (K / 32);
  if (nblocks == 0) return BSFP8_OK;
  const int64_t threads = nblocks * 2;
  hipLaunchKernelGGL(make_twin_row32_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, w,
                     nblocks, q, e, ok, bad);
  return hip_status(hipGetLastError());
}

int launch_pad_k_weight(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                        int64_t K_pad, uint8_t* q_pad, uint8_t* e_pad, hipStream_t stream) {
  const int64_t rows = G * N;
  if (rows == 0) return BSFP8_OK;
  hipLaunchKernelGGL(pad_codes_kernel, dim3(grid_for(rows * (K_pad / 16), 256)), dim3(256), 0,
                     stream, q, rows, K, K_pad, q_pad);
  hipLaunchKernelGGL(pad_exps_kernel, dim3(grid_for((rows / 32) * (K_pad / 32), 256)), dim3(256),
                     0, stream, e, rows / 32, K / 32, K_pad / 32, e_pad);
  return hip_status(hipGetLastError());
}

int launch_pad_k_input(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t K,
                       int64_t K_pad, uint16_t* x_pad, hipStream_t stream) {
  if (M == 0) return BSFP8_OK;
  const bool vec = (ldx % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x_pad) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(pad_input_vec_kernel, dim3(grid_for(M * G * K_pad / 8, 256)), dim3(256), 0,
                       stream, x, ldx, M, G, K, K_pad, x_pad);
  else
    hipLaunchKernelGGL(pad_input_scalar_kernel, dim3(grid_for(M * G * K_pad, 256)), dim3(256), 0,
                       stream, x, ldx, M, G, K, K_pad, x_pad);
  return hip_status(hipGetLastError());
}

int launch_dequant(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K, uint16_t* w,
                   hipStream_t stream) {
  const int64_t rows = G * N;
  if (rows == 0 || K == 0) return BSFP8_OK;
  // row ranges of whole 32-row blocks, each under 2^30 codes, so the kernel's indices fit 32 bits
  // (K <= 2^24, checked by the caller)
  int64_t span = ((int64_t)1 << 30) / K / 32 * 32;
  if (span < 32) span = 32;
  const uint32_t per_row = (uint32_t)(K / 8);
  const FastDiv row_of = make_fastdiv(per_row);
  for (int64_t r0 = 0; r0 < rows; r0 += span) {
    const int64_t nr = rows - r0 < span ? rows - r0 : span;
    const uint32_t npieces = (uint32_t)(nr * (K / 8));
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(npieces, 256 * DQ_UNROLL)), dim3(256), 0, stream,
                       q + r0 * K, e + (r0 / 32) * (K / 32), npieces, per_row, row_of, (uint32_t)K, w + r0 * K);
    const int st = hip_status(hipGetLastError());
    if (st != BSFP8_OK) return st;
  }
  return BSFP8_OK;
}

}  // namespace bsfp8
