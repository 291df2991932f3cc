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
// Two forms:
//  * reduce_quantize_mx_kernel, after any GEMM plan that leaves its fp32 results (or the partials
//    of its splits) in the workspace: eight lanes per 32-value block, four values (one 16-byte
//    load per partial) each, so a wave reads one contiguous kilobyte of every partial; the block
//    maximum by three lane exchanges; each lane stores its four codes as one dword and the first
//    lane of a block its scale byte. At decode sizes this second launch and the round trip of the
//    fp32 sums through memory cost more than the GEMM's own arithmetic.
//  * decode_mxfp8_kernel, the fused form for the decode plans with one split: the decode kernel's
//    waves, chunks and order of sums (gemm.hip), with 32 weight rows per workgroup so that each
//    MX block of 32 output columns is finished inside one workgroup. LDS holds every byte in
//    flight, and 32 rows of weights plus the X rows do not fit at once; so the first 16-row tile
//    streams in with the X rows as in the decode kernel, plus the first chunk of the second tile;
//    once every wave has copied its X fragments into registers, the X rows' LDS takes the second
//    tile's other chunks. The fp32 sums are bitwise those of the 16-row decode plan, so the codes
//    equal the two-kernel form's.

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
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = fminf(fmaxf(ldexpf(v[i], -s), -448.f), 448.f);   // saturating
  uint32_t codes = e4m3x4(sv[0], sv[1], sv[2], sv[3]);
  if (nonfinite) {
    codes = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) codes |= ((u[i] >> 31) ? 0xFFu : 0x7Fu) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<uint32_t*>(yq + blk * EP_BLOCK + sub * 4) = codes;
    if (sub == 0) ys[blk] = nonfinite ? (uint8_t)255 : (uint8_t)(s + 127);
  }
}

struct DecodeMxParams {
  const uint16_t* x;
  const uint8_t* q;
  const uint8_t* e;
  uint8_t* yq;                            // codes [M][G*N]
  uint8_t* ys;                            // scale bytes [M][G*N/32]
  int64_t ldx;
  uint32_t x_bytes, q_bytes, e_bytes;
  int M, G, N, K, kchunks, mblocks, nblocks, nwg;
  FastDiv dm, dn;                         // division by mblocks and nblocks
};

// Fused decode GEMM + MXFP8 epilogue: a workgroup computes rows m0 .. m0+7 of X against 32 weight
// rows n0 .. n0+31 (one block row, tiles A = rows 0..15 and B = rows 16..31) over the whole K
// range (K a multiple of 128, at most NWK*CW chunks), NWK waves along K with CW chunks each
// (chunk wk + j*NWK for wave wk, ascending j), and quantises the 32 sums of each row to one MX
// block. Loads, in issue order per wave, all in the buffer loads' LDS mode:
//   exponent words of the block row (wave 0), the wave's share of the X rows (1 KB pieces),
//   tile A's CW chunks, tile B's chunk 0;   -- wait for X, barrier, X fragments to VGPRs, barrier --
//   tile B's chunks 1 .. CW-1 into the X rows' LDS.
// The wave then computes A_0 .. A_{CW-1}, B_0 .. B_{CW-1}, each once its own loads have landed
// (loads complete in order, so the wait for chunk i is "at most the loads issued after it").
template <int NWK, int CW>
__global__ void __launch_bounds__(WAVE * NWK) decode_mxfp8_kernel(DecodeMxParams p) {
  constexpr int XR = 8;                             // rows of X per workgroup
  constexpr int TG = 128;                           // granules of one 16-row tile's chunk
  constexpr int PCH = NWK * CW;
  constexpr int ROWG = PCH * 16 + 1;                // granules per X row (one of padding)
  constexpr int XI = XR * PCH / 4;                  // X loads of 1 KB
  constexpr int XPW = XI / NWK;
  constexpr int LATE = 2 * (CW - 1);                // tile B loads issued after the X copy
  static_assert(XI % NWK == 0 && XPW >= 1, "every wave issues the same X loads");
  static_assert(PCH <= 64, "one exponent word per lane and chunk");
  static_assert(NWK * (CW - 1) * TG <= XR * ROWG, "tile B's later chunks fit the X rows' LDS");
  static_assert(CW >= 1 && CW <= 8 && XPW + 2 * CW + 2 + 1 <= 63, "vector memory counter range");
  __shared__ uint4 x_lds[XR * ROWG];                // X rows; later tile B's chunks 1 .. CW-1
  __shared__ uint4 wa_lds[NWK * CW * TG];           // tile A's chunks; at the end the K sums
  __shared__ uint4 wb_lds[NWK * TG];                // tile B's chunk 0
  __shared__ uint32_t e_lds[64];

  asm volatile("" ::"s"(p.x), "s"(p.q), "s"(p.e), "s"(p.yq), "s"(p.ys), "s"(p.ldx));
  asm volatile("" ::"s"(p.x_bytes), "s"(p.q_bytes), "s"(p.e_bytes), "s"(p.M), "s"(p.G), "s"(p.N), "s"(p.K));
  asm volatile("" ::"s"(p.kchunks), "s"(p.mblocks), "s"(p.nblocks), "s"(p.nwg));
  asm volatile("" ::"s"(p.dm.mul), "s"(p.dm.shift), "s"(p.dn.mul), "s"(p.dn.shift));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wk = wave;
  const int q4 = lane >> 4, r16 = lane & 15;
  int t = xcd_logical(blockIdx.x, p.nwg);
  int tq = fdiv(t, p.dm);
  const int mb = t - tq * p.mblocks;
  t = tq;
  tq = fdiv(t, p.dn);
  const int nb = t - tq * p.nblocks;
  const int g = tq;
  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * 32, m0 = mb * XR;
  const int c_end = p.kchunks;                      // one split: chunks 0 .. kchunks-1
  const int KB = K / 32;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // (1) exponent words of block row (g, n0/32): lane l the word of chunk l
  if (wave == 0) {
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32) * KB + lane * 4);
    lds_load4(re, lds_addr(e_lds), lane < c_end ? off : OOB);
  }
  // (2) X rows m0 .. m0+7: load i covers row i / (PCH/4), granules 64*(i % (PCH/4)) .. +63
#pragma unroll
  for (int u = 0; u < XPW; ++u) {
    const int i = wave + u * NWK;
    const int row = i / (PCH / 4), pc = i % (PCH / 4);
    const int m = m0 + row;
    const int k = (pc * 64 + lane) * 8;
    const uint32_t off = (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + k) * 2);
    if (m < M) lds_load16(rx, lds_addr(x_lds + row * ROWG + pc * 64), k < c_end * KCH ? off : OOB);
  }
  // (3) weight chunks: load (chunk c, 8-row group v) of a tile fills row R = 8v + lane/8, slot
  //     lane%8 with granule (lane%8) ^ (R/2 % 8), as in the decode kernel
  const int R0 = lane >> 3;
  const uint32_t qa = (uint32_t)(g * N + n0 + R0) * (uint32_t)K;
  const uint32_t qb = qa + 16u * (uint32_t)K;
  auto load_chunk = [&](uint32_t qrow, int c, uint4* slot) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int R = 8 * v + R0;
      const int gsrc = (lane & 7) ^ ((R >> 1) & 7);
      const uint32_t off = qrow + (uint32_t)(8 * v * K + c * KCH + gsrc * 16);
      lds_load16_stream(rq, lds_addr(slot + v * 64), c < c_end ? off : OOB);
    }
  };
  uint4* const wa = wa_lds + wave * CW * TG;
#pragma unroll
  for (int j = 0; j < CW; ++j) load_chunk(qa, wk + j * NWK, wa + j * TG);
  load_chunk(qb, wk, wb_lds + wave * TG);
  wait_vmcnt_le<2 * CW + 2>();                      // this wave's exponent and X loads
  lds_barrier();                                    // ... everyone's

  // (4) this wave's X fragments into registers, then the X rows' LDS is free for tile B
  const uint4* xrow = x_lds + (r16 & (XR - 1)) * ROWG;   // rows beyond XR feed unused columns
  uint4 xf[CW][4];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int cl = wk + j * NWK;
    xf[j][0] = xrow[cl * 16 + 2 * q4];
    xf[j][1] = xrow[cl * 16 + 2 * q4 + 1];
    xf[j][2] = xrow[cl * 16 + 8 + 2 * q4];
    xf[j][3] = xrow[cl * 16 + 9 + 2 * q4];
  }
  lds_barrier();
  uint4* const wb = x_lds + wave * (CW - 1) * TG;   // tile B's chunk j >= 1 at wb + (j-1)*TG
#pragma unroll
  for (int j = 1; j < CW; ++j) load_chunk(qb, wk + j * NWK, wb + (j - 1) * TG);

  // (5) dequant + MFMA in the decode kernel's order, tile A then tile B (the block factors of
  //     the wave's chunks are read once: both tiles lie in one block row)
  const uint8_t* eb = reinterpret_cast<const uint8_t*>(e_lds);
  const int wsw = (r16 >> 1) & 7;
  float scf[CW][2];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int cl = wk + j * NWK;
    scf[j][0] = block_scale(eb[cl * 4 + (q4 >> 1)]);
    scf[j][1] = block_scale(eb[cl * 4 + 2 + (q4 >> 1)]);
  }
  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  auto chunk = [&](int ts, int j, const uint4* slot) {
    const int cl = wk + j * NWK;
    if (cl >= c_end) return;                        // not loaded: nothing defined in LDS
    const float sc0 = scf[j][0], sc1 = scf[j][1];
    const uint4* wt = slot + r16 * 8;
    const uint4 a = wt[q4 ^ wsw], b = wt[(4 + q4) ^ wsw];
    f32x4_t c = acc[ts];
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.x, a.y, sc0), __builtin_bit_cast(bf16x8_t, xf[j][0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.z, a.w, sc0), __builtin_bit_cast(bf16x8_t, xf[j][1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.x, b.y, sc1), __builtin_bit_cast(bf16x8_t, xf[j][2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.z, b.w, sc1), __builtin_bit_cast(bf16x8_t, xf[j][3]), c, 0, 0, 0);
    acc[ts] = c;
  };
  // outstanding now, oldest first: A_0 .. A_{CW-1} (2 each), B_0 (2), B_1 .. B_{CW-1} (2 each)
  auto step = [&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (j < CW) {
      wait_vmcnt_le<2 * CW + 2 + LATE - 2 * (j + 1)>();
      chunk(0, j, wa + j * TG);
    } else if constexpr (j < 2 * CW) {
      constexpr int jb = j - CW;
      wait_vmcnt_le<LATE - 2 * jb>();
      chunk(1, jb, jb == 0 ? wb_lds + wave * TG : wb + (jb - 1) * TG);
    }
  };
  step(std::integral_constant<int, 0>{});   step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});   step(std::integral_constant<int, 3>{});
  step(std::integral_constant<int, 4>{});   step(std::integral_constant<int, 5>{});
  step(std::integral_constant<int, 6>{});   step(std::integral_constant<int, 7>{});
  step(std::integral_constant<int, 8>{});   step(std::integral_constant<int, 9>{});
  step(std::integral_constant<int, 10>{});  step(std::integral_constant<int, 11>{});
  step(std::integral_constant<int, 12>{});  step(std::integral_constant<int, 13>{});
  step(std::integral_constant<int, 14>{});  step(std::integral_constant<int, 15>{});

  // (6) waves along K: ascending-order sum through LDS (wave wk > 0 parks its sums in its own
  //     tile-A slots, which only it has read)
  if constexpr (NWK > 1) {
    f32x4_t* red = reinterpret_cast<f32x4_t*>(wa);
    if (wk > 0) {
      red[lane] = acc[0];
      red[WAVE + lane] = acc[1];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int w = 1; w < NWK; ++w) {
      const f32x4_t* rw = reinterpret_cast<const f32x4_t*>(wa_lds + w * CW * TG);
      acc[0] += rw[lane];
      acc[1] += rw[WAVE + lane];
    }
  }
  // (7) MX block of row m = m0 + r16: lane (r16, q4) holds columns q4*4 .. +3 (tile A) and
  //     16 + q4*4 .. +3 (tile B); the four lanes of a row are r16 + 16*q4
  uint32_t c_lo, c_hi;
  const uint8_t sb = mx_block_codes(acc[0], acc[1], c_lo, c_hi);
  const int m = m0 + r16;
  if (r16 < XR && m < M) store_mx_block(p.yq, p.ys, m, g, G, N, n0, q4, c_lo, c_hi, sb);
}

}  // namespace

// The fused decode form for a plan of the 16-row decode kernel with one split (8 rows of X, one
// tile per wave, 32x32 exponents). Returns BSFP8_EINVAL when the plan is not of that form.
int launch_decode_mxfp8(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                        const uint8_t* e, uint8_t* yq, uint8_t* ys, hipStream_t stream) {
  int info[8];
  if (gemm_config_info(p.cfg, info) != BSFP8_OK) return BSFP8_EINVAL;
  const int BM = info[0], NB = info[1], CW = info[3], NWN = info[4], NWK = info[5], kind = info[6];
  if (kind != 4 || (info[7] & 1) != 0 || BM != 8 || NB != 16 || NWN != 1 || p.splits != 1) return BSFP8_EINVAL;
  if (s.K % KCH != 0 || s.N % 32 != 0 || p.kchunks > NWK * CW) return BSFP8_EINVAL;
  void (*fn)(DecodeMxParams);
  if (NWK == 8 && CW == 4) fn = decode_mxfp8_kernel<8, 4>;
  else if (NWK == 4 && CW == 2) fn = decode_mxfp8_kernel<4, 2>;
  else return BSFP8_EINVAL;
  DecodeMxParams k{};
  k.x = x;
  k.q = q;
  k.e = e;
  k.yq = yq;
  k.ys = ys;
  k.ldx = s.ldx;
  const int64_t xb = ((int64_t)(s.M - 1) * s.ldx + (int64_t)s.G * s.K) * 2;
  const int64_t qb = (int64_t)s.G * s.N * s.K;
  const int64_t eb = (int64_t)s.G * (s.N / 32) * (s.K / 32);
  if (xb >= (int64_t)OOB || qb >= (int64_t)OOB || eb >= (int64_t)OOB) return BSFP8_ESHAPE;
  k.x_bytes = (uint32_t)xb;
  k.q_bytes = (uint32_t)qb;
  k.e_bytes = (uint32_t)eb;
  k.M = s.M;
  k.G = s.G;
  k.N = s.N;
  k.K = s.K;
  k.kchunks = p.kchunks;
  k.mblocks = (s.M + 7) / 8;
  k.nblocks = s.N / 32;
  k.dm = make_fastdiv((uint32_t)k.mblocks);
  k.dn = make_fastdiv((uint32_t)k.nblocks);
  const long long nwg = (long long)k.mblocks * k.nblocks * s.G;
  if (nwg <= 0 || nwg > 0x7fffffffLL) return BSFP8_ESHAPE;
  k.nwg = (int)nwg;
  hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(WAVE * NWK), 0, stream, k);
  return hip_status(hipGetLastError());
}

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
