// MXFP8 output epilogue for gfx950 (MI355X): a fixed-order fp32 sum of split partials followed by
// MXFP8 quantisation of the sum, in one pass over the partials.
//
// Page "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py" (module docstring; `install`: the
// dropped-weight path and small_mx) hands the fp32 split partials [S][M][G][N] of the partial
// kernel to one kernel that sums them and quantises the result to MXFP8, the output production
// consumes. The quantiser is the OCP MX v1.0 MXFP8 rule of quantize_mx_kernel (mx.hip), here on
// fp32 values: the scale exponent is read off the fp32 exponent field of the block maximum, which
// has the same bias as bf16's.
//
// Design: eight lanes per 32-value block, four values (one 16-byte load per partial) each, so a
// wave reads one contiguous kilobyte of every partial; the block maximum by three lane exchanges;
// each lane stores its four codes as one dword and the first lane of a block its scale byte. The
// work is a few tens of kilobytes at decode sizes, so the launch, not the bytes, is what it costs.

#include "device.h"

namespace bsfp8 {
namespace {

constexpr int EP_BLOCK = 32;                        // MX block: 32 consecutive values of a row
constexpr int EP_MAX_PARTIALS = 64;

// Sum of the S partials of one lane's four values in the pairwise order over the split index
// (the one-pass kernels' exchange tree): partial s is pushed on a stack of block sums, and while
// the top of the stack holds a block of the same size the two are added, so aligned blocks of
// 2, 4, 8, ... partials are summed as perfect trees; at the end the blocks left on the stack are
// added from the right (an unpaired block is carried up unchanged by every level). The loop is
// unrolled, so the stack height before partial s (popcount(s)) and the number of merges after it
// (the trailing zeros of s + 1) are constants and the stack lives in registers.
__device__ __forceinline__ f32x4_t sum_pairwise(const f32x4_t* p, int64_t stride, int S) {
  f32x4_t stk[7];
#pragma unroll
  for (int s = 0; s < EP_MAX_PARTIALS; ++s) {
    if (s < S) {
      f32x4_t v = p[(int64_t)s * stride];
      const int h = __builtin_popcount(s);
      const int merges = __builtin_ctz(s + 1);
#pragma unroll
      for (int j = 0; j < merges; ++j) v = stk[h - 1 - j] + v;
      stk[h - merges] = v;
    }
  }
  const int height = __builtin_popcount(S);
  f32x4_t acc = stk[0];
  bool have = false;
#pragma unroll
  for (int i = 6; i >= 0; --i) {
    if (i < height) {
      acc = have ? stk[i] + acc : stk[i];
      have = true;
    }
  }
  return acc;
}

__device__ __forceinline__ f32x4_t sum_ascending(const f32x4_t* p, int64_t stride, int S) {
  f32x4_t acc = p[0];
  for (int s = 1; s < S; ++s) acc = acc + p[(int64_t)s * stride];
  return acc;
}

template <int ORDER>
__global__ void __launch_bounds__(256) reduce_quantize_mx_kernel(const float* __restrict__ part, int S,
                                                                 int64_t ml, int64_t nblk,
                                                                 uint8_t* __restrict__ yq,
                                                                 uint8_t* __restrict__ ys) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 3;                       // 32-value block; eight lanes each
  const int sub = (int)(t & 7);
  const bool live = blk < nblk;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part) + blk * 8 + sub;
    const int64_t stride = ml / 4;                  // f32x4 elements per partial
    v = ORDER == BSFP8_SUM_PAIRWISE ? sum_pairwise(p, stride, S) : sum_ascending(p, stride, S);
  }
  uint32_t u[4], amax = 0, nonfinite = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u[i] = __float_as_uint(v[i]);
    const uint32_t mag = u[i] & 0x7FFFFFFFu;
    nonfinite |= mag >= 0x7F800000u ? 1u : 0u;
    amax = mag > amax ? mag : amax;
  }
  // the eight lanes of a block are adjacent in the wave (dead lanes hold zeros)
#pragma unroll
  for (int off = 1; off <= 4; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)amax, off);
    amax = o > amax ? o : amax;
    nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off);
  }
  // floor(log2(amax)) = E - 127 for a normal fp32 maximum; a zero or subnormal maximum gives the
  // smallest scale. s = floor(log2(amax)) - 8, clamped below at -127 (above, E <= 254 keeps
  // s <= 119). Every scaled value is then below 512 in magnitude, and exact: the scaling is a
  // power of two, and a value that falls below the fp32 normals is far below e4m3's 2^-10.
  const int E = (int)(amax >> 23);
  int s = E == 0 ? -127 : E - 135;
  s = s < -127 ? -127 : s;
  uint32_t codes = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c;
    if (nonfinite) {
      c = (u[i] >> 31) ? 0xFFu : 0x7Fu;
    } else {
      float sv = ldexpf(v[i], -s);
      sv = fminf(fmaxf(sv, -448.f), 448.f);         // saturating conversion
      c = e4m3_rne(sv);
    }
    codes |= c << (8 * i);
  }
  if (live) {
    *reinterpret_cast<uint32_t*>(yq + blk * EP_BLOCK + sub * 4) = codes;
    if (sub == 0) ys[blk] = nonfinite ? (uint8_t)255 : (uint8_t)(s + 127);
  }
}

}  // namespace

int launch_reduce_quantize_mx(const float* part, int S, int64_t M, int64_t L, int order, uint8_t* yq,
                              uint8_t* ys, hipStream_t stream) {
  if (S < 1 || S > EP_MAX_PARTIALS || L % EP_BLOCK) return BSFP8_EINVAL;
  const int64_t nblk = M * (L / EP_BLOCK);
  if (nblk == 0) return BSFP8_OK;
  const int64_t threads = nblk * 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (order == BSFP8_SUM_PAIRWISE)
    hipLaunchKernelGGL(reduce_quantize_mx_kernel<BSFP8_SUM_PAIRWISE>, grid, dim3(256), 0, stream, part, S,
                       M * L, nblk, yq, ys);
  else
    hipLaunchKernelGGL(reduce_quantize_mx_kernel<BSFP8_SUM_ASCENDING>, grid, dim3(256), 0, stream, part, S,
                       M * L, nblk, yq, ys);
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
