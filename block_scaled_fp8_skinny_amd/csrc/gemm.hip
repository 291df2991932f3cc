// Small-M block-scaled fp8 weight GEMM for gfx950 (MI355X).
//
// Computes Y[m][g][n] = sum_k X[m][g*K + k] * W[g][n][k], where the weight is stored as e4m3
// codes plus one exponent byte per 32x32 block and each tile is rebuilt exactly in bf16
// registers before a bf16 MFMA with fp32 accumulation (page
// "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py": kernels _wo_a_partial_w8 and
// _wo_a_mid_kernel; its notes ask that split-K partials be summed in a fixed order).
//
// Design (gfx950, wave64):
//  * MFMA v_mfma_f32_16x16x32_bf16 with the WEIGHT as the A operand (16 rows of W) and X^T as
//    the B operand (16 rows of X): D[n][m] holds four consecutive n per lane.
//  * K is walked in 128-wide chunks. In a chunk, lane (q, r) of the MFMA takes the k values
//    16*q .. 16*q + 15 and 64 + 16*q .. 64 + 16*q + 15 of its row r (q = lane/16) in every kernel,
//    so a chunk's four MFMAs sum the same products in the same order whichever kernel runs it.
//  * How they arrive: the first kernels (gemm_kernel, gemm_direct_kernel) load the weight pieces
//    in that lane order straight from HBM into VGPRs (64 contiguous bytes per row and load); the
//    decode, paired, LDS-staged register and tile kernels read eight lanes per row (128
//    contiguous bytes per row and load, which HBM streams about 30% faster) straight into LDS
//    with the buffer loads' LDS mode, each lane fetching the granule that belongs in its slot of
//    a swizzled row-major tile, and take the MFMA fragments from there.
//  * Every global load is a raw buffer load: out-of-range offsets return zero, so masked
//    pieces (ragged K tail, rows beyond M) need no branches, and each wave waits for exactly the
//    loads a chunk needs (the compiler's counts for VGPR loads, explicit s_waitcnt for LDS-mode
//    loads, which complete in order). Dequant and MFMA of the first chunks therefore overlap the
//    arrival of the later ones.
//  * Dequant is v_cvt_scalef32_pk_bf16_fp8: 2 codes -> 2 bf16 scaled by the block factor in one
//    instruction, exact for every code and exponent byte 0..254 (checked on the hardware).
//  * X rows and the exponent bytes are staged in LDS in layouts whose fragment reads are free of
//    bank conflicts. Rows at or beyond M are not loaded: they feed only MFMA output columns that
//    are never stored.
//  * Waves of a workgroup split the n rows (NWN) and the chunks (NWK); the NWK partial tiles are
//    summed through LDS in ascending wave order. Workgroups may further split K (splits > 1).
//    Their partials meet in a binary tree of pairwise combines: at each node the two partners
//    swap their fp32 value into one 64-bit slot with an atomic exchange; the second to arrive
//    gets the first one's value back, adds (a + b == b + a exactly in IEEE arithmetic, so the
//    sum does not depend on who arrives first), clears the slot for the next call and carries
//    the sum to the parent node. The tree's shape is fixed by the split index, so every output
//    is bitwise reproducible, and the exchange carries the data itself: no counters, no fences,
//    no waiting for stores to drain.
//  * The map chunk -> (split, pass, wave, step) depends only on the chunk index and the plan,
//    not on K, so zero-padding K inside the same chunk count leaves every fp32 sum unchanged.
//  * Workgroup ids of the flat-grid kernels are remapped so that consecutive logical tiles run on
//    the same XCD (workgroups are dealt round-robin over the 8 XCDs): splits sharing an X slab
//    and m-blocks sharing a weight tile hit the same L2. The decode kernels take their tile from
//    a three-dimensional grid instead (no index arithmetic before the first loads).

#include <type_traits>

#include "device.h"

namespace bsfp8 {
namespace {


template <int MT, int NT, int NWN, int NWK, int CW>
__global__ void __launch_bounds__(WAVE * NWN * NWK)
gemm_kernel(KParams p) {
  constexpr int NTHR = WAVE * NWN * NWK;
  constexpr int BM = 16 * MT;
  constexpr int NB = 16 * NT * NWN;
  constexpr int PCH = NWK * CW;                     // chunks per pass
  constexpr int XSLOTS = PCH * 4 * MT * WAVE;       // 16-byte X fragment slots of one pass
  constexpr int XBYTES = XSLOTS * 16;
  constexpr int EROWS = NB >= 32 ? NB / 32 : 1;
  constexpr int ECOLS = PCH * 4;
  static_assert(XSLOTS % NTHR == 0, "X staging must divide evenly over the threads");
  static_assert(EROWS * ECOLS <= NTHR, "one exponent byte per thread");
  constexpr int XPT = XSLOTS / NTHR;
  constexpr int REDBYTES = (NWK - 1) * NWN * MT * NT * WAVE * 16;
  static_assert(REDBYTES <= XBYTES, "the wave reduction aliases the X buffer");

  __shared__ __attribute__((aligned(16))) uint8_t x_lds[XBYTES];
  __shared__ uint8_t e_lds[EROWS * ECOLS];

  prefetch_args_only(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wk = wave / NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int npass = (c_end - c_begin + PCH - 1) / PCH;
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // weight rows of this lane (+16*ts): byte offset of the row start in q
  const int nrow = n0 + wn * 16 * NT + r16;
  const uint32_t qrow = (uint32_t)(g * N + nrow) * (uint32_t)K;
  const int erow0 = n0 / 32;
  const uint32_t ebase = (uint32_t)(g * (N / 32) + erow0) * (uint32_t)KB;

  // ---- loaders (all branch-free; masked pieces read as zero) ----
  auto load_x = [&](int pass, uint4 (&xr)[XPT]) {
    const int pc0 = c_begin + pass * PCH;
    const int pch = min(PCH, c_end - pc0);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int f = tid + i * NTHR;
      const int blk = f >> 6, L = f & 63;
      const int cp = blk / (4 * MT), jj = (blk / MT) & 3, mt = blk % MT;
      const int m = m0 + mt * 16 + (L & 15);
      const int k = (pc0 + cp) * KCH + (jj >> 1) * 64 + (L >> 4) * 16 + (jj & 1) * 8;
      const bool ok = m < M && cp < pch && k < K;
      const uint32_t off = (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + k) * 2);
      xr[i] = load16(rx, ok ? off : OOB);
    }
  };
  auto load_e = [&](int pass) -> uint32_t {
    const int pc0 = c_begin + pass * PCH;
    const int pch = min(PCH, c_end - pc0);
    const int er = tid / ECOLS, ec = tid % ECOLS;
    const int kb = pc0 * 4 + ec;
    const bool ok = tid < EROWS * ECOLS && ec < pch * 4 && kb < KB;
    const uint32_t off = ebase + (uint32_t)(er * KB + kb);
    return __builtin_amdgcn_raw_buffer_load_b8(re, (int)(ok ? off : OOB), 0, 0);
  };
  auto load_w = [&](int pass, uint4 (&wr)[CW][NT][2]) {
    const int pc0 = c_begin + pass * PCH;
    const int pch = min(PCH, c_end - pc0);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int cp = wk + j * NWK;
#pragma unroll
      for (int ts = 0; ts < NT; ++ts)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = (pc0 + cp) * KCH + h * 64 + q4 * 16;
          const bool ok = cp < pch && k < K;
          wr[j][ts][h] = load16_stream(rq, ok ? qrow + (uint32_t)(ts * 16 * K + k) : OOB);
        }
    }
  };
  auto stage = [&](int pass, const uint4 (&xr)[XPT], uint32_t ev) {
    if (pass) __syncthreads();                      // the previous pass is fully consumed
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int f = tid + i * NTHR;
      const int mt = (f >> 6) % MT;
      if (m0 + mt * 16 + (f & 15) < M) *reinterpret_cast<uint4*>(x_lds + f * 16) = xr[i];
    }
    if (tid < EROWS * ECOLS) e_lds[tid] = (uint8_t)ev;
    __syncthreads();
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int pass, const uint4 (&wr)[CW][NT][2]) {
    const int pc0 = c_begin + pass * PCH;
    const int pch = min(PCH, c_end - pc0);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int cp = wk + j * NWK;
      if (cp < pch) {
#pragma unroll
        for (int ts = 0; ts < NT; ++ts) {
          const int er = (nrow + ts * 16) / 32 - erow0;
          const float sc0 = block_scale(e_lds[er * ECOLS + cp * 4 + (q4 >> 1)]);
          const float sc1 = block_scale(e_lds[er * ECOLS + cp * 4 + 2 + (q4 >> 1)]);
          const uint4 a = wr[j][ts][0], b = wr[j][ts][1];
          const bf16x8_t w0 = dequant8(a.x, a.y, sc0);
          const bf16x8_t w1 = dequant8(a.z, a.w, sc0);
          const bf16x8_t w2 = dequant8(b.x, b.y, sc1);
          const bf16x8_t w3 = dequant8(b.z, b.w, sc1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint8_t* fb = x_lds + ((cp * 4 * MT + mt) * 64 + lane) * 16;
            const bf16x8_t x0 = *reinterpret_cast<const bf16x8_t*>(fb);
            const bf16x8_t x1 = *reinterpret_cast<const bf16x8_t*>(fb + MT * 1024);
            const bf16x8_t x2 = *reinterpret_cast<const bf16x8_t*>(fb + 2 * MT * 1024);
            const bf16x8_t x3 = *reinterpret_cast<const bf16x8_t*>(fb + 3 * MT * 1024);
            f32x4_t c = acc[mt][ts];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, x2, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, x3, c, 0, 0, 0);
            acc[mt][ts] = c;
          }
        }
      }
    }
  };

  // ---- main loop: two register sets for the weights, next pass prefetched ----
  uint4 xr[XPT];
  uint4 wa[CW][NT][2], wb[CW][NT][2];
  load_x(0, xr);                                    // X first (L2-resident), then exponents,
  uint32_t ev = load_e(0);                          // then the HBM weight stream
  load_w(0, wa);
  for (int pass = 0; pass < npass; pass += 2) {
    stage(pass, xr, ev);
    if (pass + 1 < npass) {
      load_x(pass + 1, xr);
      ev = load_e(pass + 1);
      load_w(pass + 1, wb);
    }
    compute(pass, wa);
    if (pass + 1 >= npass) break;
    stage(pass + 1, xr, ev);
    if (pass + 2 < npass) {
      load_x(pass + 2, xr);
      ev = load_e(pass + 2);
      load_w(pass + 2, wa);
    }
    compute(pass + 1, wb);
  }

  // Sum the NWK waves' tiles in ascending wave order (through LDS, aliasing the X buffer).
  if constexpr (NWK > 1) {
    __syncthreads();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(x_lds);
    if (wk > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ts = 0; ts < NT; ++ts)
          red[((((wk - 1) * NWN + wn) * MT + mt) * NT + ts) * WAVE + lane] = acc[mt][ts];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int w = 1; w < NWK; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ts = 0; ts < NT; ++ts)
          acc[mt][ts] += red[((((w - 1) * NWN + wn) * MT + mt) * NT + ts) * WAVE + lane];
  }

  if (p.splits == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + mt * 16 + r16;
      if (m < M) {
#pragma unroll
        for (int ts = 0; ts < NT; ++ts) {
          const int n = n0 + wn * 16 * NT + ts * 16 + q4 * 4;
          const size_t off = ((size_t)m * G + g) * N + n;
          const f32x4_t v = acc[mt][ts];
          if (p.out_f32) {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + off) = v;
          } else {
            const uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + off) = o;
          }
        }
      }
    }
    return;
  }

  // splits > 1: pairwise-combine tree over the split index.
  constexpr int NV = MT * NT * 4;
  float v[NV];
  size_t off[NV];
  int mr[NV];
  bool live[NV];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (mt * NT + ts) * 4 + r;
        const int m = m0 + mt * 16 + r16;
        const int n = n0 + wn * 16 * NT + ts * 16 + q4 * 4 + r;
        v[i] = acc[mt][ts][r];
        off[i] = ((size_t)m * G + g) * N + n;
        mr[i] = m;
        live[i] = m < M;
      }
  combine_splits<NV>(p, s, v, off, mr, live);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (live[i]) store_out(p, off[i], v[i]);
}

// Small-M kernel (at most 16 rows of X per workgroup, one pass over its K range). The weight
// pieces go straight from HBM into the lane's MFMA registers. The workgroup's X rows (only the
// rows below M) and exponent bytes are first loaded densely and coalesced, once per workgroup,
// into LDS: X row-major with a 16-byte pad per row, so both the row-wise writes and the
// fragment reads (16 rows at one k per 16 lanes) hit distinct banks. These L2-resident loads are
// issued before the weight stream; each chunk's dequant + MFMA then waits only for its own
// weight pieces. Each wave owns the chunks wk, wk + NWK, ... of the workgroup's range, so an
// output's fp32 sum is the same ascending chain of chunks as in gemm_kernel with the same NWK
// and chunks per split.
template <int NT, int NWN, int NWK, int CW>
__global__ void __launch_bounds__(WAVE * NWN * NWK)
gemm_direct_kernel(KParams p) {
  constexpr int NTHR = WAVE * NWN * NWK;
  constexpr int NB = 16 * NT * NWN;
  constexpr int PCH = NWK * CW;                     // chunks of the workgroup
  constexpr int ROWB = PCH * KCH * 2 + 16;          // LDS bytes per X row (padded)
  constexpr int XPIECES = 16 * PCH * 16;            // 16-byte pieces of 16 full rows
  constexpr int XPT = (XPIECES + NTHR - 1) / NTHR;
  constexpr int EROWS = NB >= 32 ? NB / 32 : 1;
  constexpr int ECOLS = PCH * 4;
  static_assert(EROWS * ECOLS <= NTHR, "one exponent byte per thread");
  constexpr int RED = NWK > 1 ? (NWK - 1) * NWN * NT * WAVE : 1;
  __shared__ __attribute__((aligned(16))) uint8_t x_lds[16 * ROWB];
  __shared__ uint8_t e_lds[EROWS * ECOLS];
  __shared__ f32x4_t red[RED];

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wk = wave / NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * NB, m0 = mb * 16;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int KB = K / 32;
  const int rows = min(16, M - m0);                 // X rows of this workgroup
  const int k_lo = c_begin * KCH;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // (1) X rows [m0, m0+rows) x k in [k_lo, k_lo + PCH*128): piece i of a row is 8 values
  // (only ceil(rows * PCH * 16 / NTHR) of the XPT load slots are issued: a uniform bound)
  const int xn = (rows * PCH * 16 + NTHR - 1) / NTHR;
  uint4 xv[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int f = tid + i * NTHR;
    const int row = f / (PCH * 16), pc = f % (PCH * 16);
    const int k = k_lo + pc * 8;
    const bool ok = f < rows * PCH * 16 && k < K && k < c_end * KCH;
    const uint32_t off = (uint32_t)(((int64_t)(m0 + row) * p.ldx + (int64_t)g * K + k) * 2);
    if (i < xn) xv[i] = load16(rx, ok ? off : OOB);
  }
  // exponent bytes: EROWS block rows x the workgroup's K blocks
  uint32_t ev;
  {
    const int er = tid / ECOLS, ec = tid % ECOLS;
    const int kb = c_begin * 4 + ec;
    const bool ok = tid < EROWS * ECOLS && kb < KB && kb < c_end * 4;
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32 + er) * KB + kb);
    ev = __builtin_amdgcn_raw_buffer_load_b8(re, (int)(ok ? off : OOB), 0, 0);
  }
  // Every wave's X and exponent requests enter the CU's memory pipeline before any weight
  // request (a bare s_barrier: it waits for no data), so they are not queued behind HBM misses.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NTHR > WAVE) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  // (2) the weight pieces (HBM)
  const int nrow = n0 + wn * 16 * NT + r16;         // + 16*ts
  const uint32_t qrow = (uint32_t)(g * N + nrow) * (uint32_t)K;
  uint4 wr[CW][NT][2];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int c = c_begin + wk + j * NWK;
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = c * KCH + h * 64 + q4 * 16;
        wr[j][ts][h] = load16_stream(rq, (c < c_end && k < K) ? qrow + (uint32_t)(ts * 16 * K + k) : OOB);
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  // (3) stage X and the exponents in LDS
  pin_epilogue_args(p);                             // the loads are issued
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int f = tid + i * NTHR;
    const int row = f / (PCH * 16), pc = f % (PCH * 16);
    if (i < xn && f < rows * PCH * 16) *reinterpret_cast<uint4*>(x_lds + row * ROWB + pc * 16) = xv[i];
  }
  if (tid < EROWS * ECOLS) e_lds[tid] = (uint8_t)ev;
  __syncthreads();
  // (4) dequant + MFMA, chunk by chunk in ascending order. Chunks beyond the range were loaded
  //     as zeros and add exact zeros; computing them unconditionally keeps every load ahead of
  //     the first MFMA. X rows at or beyond M hold stale LDS data: they feed only MFMA output
  //     columns that are never stored. Their reads stay inside the x_lds tile.
  f32x4_t acc[NT];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts) acc[ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* xrow = x_lds + r16 * ROWB + q4 * 32;
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int cl = wk + j * NWK;                    // chunk index inside the workgroup
    const bf16x8_t x0 = *reinterpret_cast<const bf16x8_t*>(xrow + cl * 256);
    const bf16x8_t x1 = *reinterpret_cast<const bf16x8_t*>(xrow + cl * 256 + 16);
    const bf16x8_t x2 = *reinterpret_cast<const bf16x8_t*>(xrow + cl * 256 + 128);
    const bf16x8_t x3 = *reinterpret_cast<const bf16x8_t*>(xrow + cl * 256 + 144);
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const int er = (nrow + ts * 16) / 32 - n0 / 32;
      const float sc0 = block_scale(e_lds[er * ECOLS + cl * 4 + (q4 >> 1)]);
      const float sc1 = block_scale(e_lds[er * ECOLS + cl * 4 + 2 + (q4 >> 1)]);
      const uint4 a = wr[j][ts][0], b = wr[j][ts][1];
      f32x4_t c = acc[ts];
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.x, a.y, sc0), x0, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.z, a.w, sc0), x1, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.x, b.y, sc1), x2, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.z, b.w, sc1), x3, c, 0, 0, 0);
      acc[ts] = c;
    }
  }
  // (5) waves along K: ascending-order sum through LDS
  if constexpr (NWK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) red[(((wk - 1) * NWN + wn) * NT + ts) * WAVE + lane] = acc[ts];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int w = 1; w < NWK; ++w)
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) acc[ts] += red[(((w - 1) * NWN + wn) * NT + ts) * WAVE + lane];
  }
  // (6) output
  const int m = m0 + r16;
  const bool mrow = m < M;
  if (p.splits == 1) {
    if (mrow) {
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int n = n0 + wn * 16 * NT + ts * 16 + q4 * 4;
        const size_t o = ((size_t)m * G + g) * N + n;
        const f32x4_t v = acc[ts];
        if (p.out_f32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = v;
        } else {
          const uint2 w2 = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
        }
      }
    }
    return;
  }
  constexpr int NV = NT * 4;
  float v[NV];
  size_t off[NV];
  int mr[NV];
  bool live[NV];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[ts * 4 + r] = acc[ts][r];
      off[ts * 4 + r] = ((size_t)m * G + g) * N + n0 + wn * 16 * NT + ts * 16 + q4 * 4 + r;
      mr[ts * 4 + r] = m;
      live[ts * 4 + r] = mrow;
    }
  combine_splits<NV>(p, s, v, off, mr, live);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (live[i]) store_out(p, off[i], v[i]);
}

// Epilogue of the register kernels (rows_kernel, rows_dma_kernel): the NWK waves along K each hold
// a partial of the whole BM x NB tile. They meet in LDS (`red`, WS f32x4 slots per wave, which
// alias each wave's own staging area, so no barrier is needed before the writes) and are added in
// ascending wave order; the tile then goes out as bf16/fp32, as MXFP8 codes, or into the
// pairwise-exchange tree of the splits.
template <int MT, int NT, int NWK, int WS>
__device__ __forceinline__ void rows_epilogue(KParams& p, f32x4_t (&acc)[MT][NT], f32x4_t* red, int wk, int lane,
                                              int m0, int n0, int g, int s) {
  constexpr int TILES = MT * NT;
  constexpr int TPW = (TILES + NWK - 1) / NWK;      // tiles summed and stored per wave
  static_assert(TILES * WAVE <= WS, "a wave's partial tiles fit in its area");
  const int q4 = lane >> 4, r16 = lane & 15;
  const int M = p.M, N = p.N, G = p.G;
  // Sum the NWK partial tiles in ascending wave order; wave w finishes tiles w, w + NWK, ...
  f32x4_t v4[TPW];
  int tix[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    tix[i] = NWK > 1 ? wk + i * NWK : i;
    v4[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (NWK > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) red[wk * WS + (mt * NT + ts) * WAVE + lane] = acc[mt][ts];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (tix[i] < TILES) {
        f32x4_t a = red[tix[i] * WAVE + lane];
#pragma unroll
        for (int w = 1; w < NWK; ++w) a += red[w * WS + tix[i] * WAVE + lane];
        v4[i] = a;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TPW; ++i) v4[i] = acc[i / NT][i % NT];
  }

  // MXFP8 output (one split): wave w finishes the 32-column blocks of strips w, w + NWK, ...,
  // adding each tile's wave partials in the same ascending order as above, and quantises them
  if (p.yq) {
    if constexpr (NT % 2 == 0) {
      constexpr int NBLK = NT / 2;
      for (int j = wk; j < MT * NBLK; j += NWK) {
        const int mt = j / NBLK, bk = j % NBLK;
        f32x4_t half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tt = mt * NT + 2 * bk + h;
          if constexpr (NWK > 1) {
            f32x4_t v = red[tt * WAVE + lane];
#pragma unroll
            for (int w = 1; w < NWK; ++w) v += red[w * WS + tt * WAVE + lane];
            half[h] = v;
          } else {
            half[h] = acc[mt][2 * bk + h];
          }
        }
        uint32_t c_lo, c_hi;
        const uint8_t sb = mx_block_codes(half[0], half[1], c_lo, c_hi);
        const int m = m0 + mt * 16 + r16;
        if (m < M) store_mx_block(p.yq, p.ys, m, g, G, N, n0 + 32 * bk, q4, c_lo, c_hi, sb);
      }
    }
    return;
  }

  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int mt = tix[i] / NT, ts = tix[i] % NT;
      const int m = m0 + mt * 16 + r16;
      if (tix[i] < TILES && m < M) {
        const size_t o = ((size_t)m * G + g) * N + n0 + ts * 16 + q4 * 4;
        const f32x4_t v = v4[i];
        if (p.out_f32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = v;
        } else {
          const uint2 w2 = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
        }
      }
    }
    return;
  }
  constexpr int NV = TPW * 4;
  float v[NV];
  size_t off[NV];
  int mr[NV];
  bool live[NV];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int mt = tix[i] / NT, ts = tix[i] % NT;
    const int m = m0 + mt * 16 + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[i * 4 + r] = v4[i][r];
      off[i * 4 + r] = ((size_t)m * G + g) * N + n0 + ts * 16 + q4 * 4 + r;
      mr[i * 4 + r] = m;
      live[i * 4 + r] = tix[i] < TILES && m < M;
    }
  }
  combine_splits<NV>(p, s, v, off, mr, live);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (live[i]) store_out(p, off[i], v[i]);
}

// Register kernel for mid row counts: BM = 16*MT rows of X and NB = 16*NT weight rows per
// workgroup, NWK waves along K, one pass over the workgroup's K range. The waves of a workgroup
// share nothing (each owns the chunks wk, wk + NWK, ...), so there is no LDS limit on the tile's
// K extent; a ring of D chunk buffers per wave keeps D chunks of loads in flight (chunk j + D is
// issued as soon as chunk j has been consumed).
//  * X is read coalesced, eight lanes per row (128 contiguous bytes per row and load). Each wave
//    then turns its chunk into the MFMA layout through a private LDS tile: 16 rows x 256 bytes
//    per 16-row block, granule g of row r at slot g ^ r, which the fragment reads (16 rows x one
//    granule) cross without bank conflicts.
//  * The weights are read eight lanes per row (128 contiguous bytes per row and load, which HBM
//    streams far better than the MFMA order's 64) and reordered through a second per-wave LDS
//    tile, row-major with granule g of row R at slot g ^ (R/2 % 8).
//  * The NWK partial tiles meet in LDS (each wave writes its own X area, so no barrier is needed
//    before) and each wave sums, in ascending wave order, and stores its share of the tiles.
template <int MT, int NT, int NWK, int CW, int D>
__global__ void __launch_bounds__(WAVE * NWK)
gemm_rows_kernel(KParams p) {
  constexpr int NTHR = WAVE * NWK;
  constexpr int BM = 16 * MT;
  constexpr int NB = 16 * NT;
  constexpr int PCH = NWK * CW;                     // chunks of the workgroup
  constexpr int EROWS = NB >= 32 ? NB / 32 : 1;
  constexpr int ECOLS = PCH * 4;
  constexpr int XG = MT * 256;                      // 16-byte granules of one wave's X chunk
  static_assert(EROWS * ECOLS <= NTHR, "one exponent byte per thread");
  static_assert(D >= 1 && D <= CW, "ring depth");
  __shared__ uint8_t e_lds[EROWS * ECOLS];
  __shared__ uint4 xs[NWK * XG];
  __shared__ uint4 wsm[NWK * NT * 128];            // each wave's weight chunk, 16 rows x 8 granules per tile

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wk = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int cr = lane >> 3, cp = lane & 7;          // coalesced X: row cr (+8), granule cp (+8)

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N;
  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // exponent bytes: EROWS block rows x the workgroup's K blocks, one per thread, issued first
  uint32_t ev;
  {
    const int er = tid / ECOLS, ec = tid % ECOLS;
    const int kb = c_begin * 4 + ec;
    const bool ok = tid < EROWS * ECOLS && kb < KB && kb < c_end * 4;
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32 + er) * KB + kb);
    ev = __builtin_amdgcn_raw_buffer_load_b8(re, (int)(ok ? off : OOB), 0, 0);
  }

  // X rows m0 + 16*mt + 8*hr + cr of this lane's coalesced loads (zero beyond M)
  uint32_t xrow[MT][2];
  bool xok[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
      const int m = m0 + mt * 16 + 8 * hr + cr;
      xok[mt][hr] = m < M;
      xrow[mt][hr] = xok[mt][hr] ? (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K) * 2) : 0u;
    }
  // weights, eight lanes per row: load v of tile ts covers rows 8v .. 8v+7, the lane takes row
  // 8v + lane/8, bytes 16*(lane%8) of the chunk
  const uint32_t qrow8 = (uint32_t)(g * N + n0 + (lane >> 3)) * (uint32_t)K;

  // Chunk j of this wave is chunk c = c_begin + wk + j*NWK. X load i covers rows 8*(i%2) .. +7 of
  // a 16-row block, k in [c*128 + 64*(i/2), +64) (eight lanes per row, 128 bytes); weight load v
  // covers the chunk's 128 bytes of 8 weight rows. Out-of-range pieces read as zero.
  struct Buf {
    uint4 w[NT][2];
    uint4 x[MT][4];
  };
  auto load = [&](int j, Buf& b) {
    const int c = c_begin + wk + j * NWK;
    const bool cok = c < c_end;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = c * KCH + 64 * (i >> 1) + 8 * cp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        b.x[mt][i] = load16(rx, cok && k < K && xok[mt][i & 1] ? xrow[mt][i & 1] + (uint32_t)k * 2 : OOB);
    }
    const int kw = c * KCH + (lane & 7) * 16;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int ts = 0; ts < NT; ++ts)
        b.w[ts][v] = load16_stream(rq, cok && kw < K ? qrow8 + (uint32_t)((ts * 16 + 8 * v) * K + kw) : OOB);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) acc[mt][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4* const xw = xs + wk * XG;                   // this wave's X area: row r, granule g at
  const int fr = r16;                               //   r*16 + (g ^ r), read by row r16
  uint4* const ww = wsm + wk * NT * 128;            // this wave's weight area: row R, granule g
  const int wr8 = lane >> 3;                        //   at R*8 + (g ^ (R/2 % 8))
  const int wsw = (r16 >> 1) & 7;
  auto compute = [&](int j, const Buf& b) {
    const int cl = wk + j * NWK;                    // chunk index inside the workgroup
    // X chunk -> LDS (row-major, swizzled) -> MFMA fragments: lane (r16, q4) takes the k values
    // 64h + 16*q4 + 8u + [0, 8) of row r16 for MFMA 2h + u, the k values of its weight piece h.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (i & 1) + cr;
        xw[mt * 256 + row * 16 + ((8 * (i >> 1) + cp) ^ row)] = b.x[mt][i];
      }
    bf16x8_t xf[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int gr = 8 * (f >> 1) + 2 * q4 + (f & 1);
        xf[mt][f] = __builtin_bit_cast(bf16x8_t, xw[mt * 256 + r16 * 16 + (gr ^ fr)]);
      }
    // weights -> LDS (row-major, swizzled) -> the MFMA order: lane (r16, q4) takes granules q4
    // and 4 + q4 of row r16
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int R = 8 * v + wr8;
        ww[(ts * 16 + R) * 8 + ((lane & 7) ^ ((R >> 1) & 7))] = b.w[ts][v];
      }
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const int er = (n0 + ts * 16 + r16) / 32 - n0 / 32;
      const float sc0 = block_scale(e_lds[er * ECOLS + cl * 4 + (q4 >> 1)]);
      const float sc1 = block_scale(e_lds[er * ECOLS + cl * 4 + 2 + (q4 >> 1)]);
      const uint4 wa = ww[(ts * 16 + r16) * 8 + (q4 ^ wsw)];
      const uint4 wb = ww[(ts * 16 + r16) * 8 + ((4 + q4) ^ wsw)];
      const bf16x8_t w0 = dequant8(wa.x, wa.y, sc0);
      const bf16x8_t w1 = dequant8(wa.z, wa.w, sc0);
      const bf16x8_t w2 = dequant8(wb.x, wb.y, sc1);
      const bf16x8_t w3 = dequant8(wb.z, wb.w, sc1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t c = acc[mt][ts];
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, xf[mt][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, xf[mt][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, xf[mt][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, xf[mt][3], c, 0, 0, 0);
        acc[mt][ts] = c;
      }
    }
  };

  // Ring of D chunk buffers; chunks beyond the range were loaded as zeros and add exact zeros,
  // so every wave runs the same straight-line sequence.
  Buf ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) load(j, ring[j]);
  pin_epilogue_args(p);                             // the first loads are issued
  __builtin_amdgcn_sched_barrier(0);
  if (tid < EROWS * ECOLS) e_lds[tid] = (uint8_t)ev;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    compute(j, ring[j % D]);
    if (j + D < CW) {
      __builtin_amdgcn_sched_barrier(0);
      load(j + D, ring[j % D]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  rows_epilogue<MT, NT, NWK, XG>(p, acc, reinterpret_cast<f32x4_t*>(xs), wk, lane, m0, n0, g, s);
}

// Register kernel with LDS-mode staging: the tiles, waves, chunk order, MFMA order and epilogue of
// gemm_rows_kernel (so the two give bitwise the same results for the same MT, NT, NWK and CW),
// but each wave streams its chunks straight from memory into a private ring of D LDS buffers with
// the buffer loads' LDS mode instead of passing them through VGPRs and LDS stores:
//  * an X chunk (BM rows x 256 bytes) is BM/4 wave loads of four 256-byte row pieces, sixteen
//    lanes per row, each lane fetching the granule that belongs in its slot (granule g of row r at
//    slot g ^ (r % 16)); a weight chunk (NB rows x 128 bytes) is NB/8 wave loads of eight 128-byte
//    row pieces (granule g of row R at slot g ^ (R/2 % 8)). Both layouts are the ones the rows
//    kernel writes, so the fragment reads are the same and conflict-free;
//  * a wave only ever reads its own buffers, so it needs no barrier: it waits for its own loads
//    (every chunk issues the same PC loads, chunks past the split's range at out-of-range
//    offsets, so the counts stay exact) and refills a buffer once its reads of it are done;
//  * chunks past the range are not computed (the accumulators start at +0 and can never hold -0,
//    so adding their zero products would change nothing).
// K must be whole 128-wide chunks.
template <int MT, int NT, int NWK, int CW, int D>
__global__ void __launch_bounds__(WAVE * NWK)
gemm_rows_dma_kernel(KParams p) {
  constexpr int BM = 16 * MT;
  constexpr int NB = 16 * NT;
  constexpr int PCH = NWK * CW;                     // chunks of the workgroup
  constexpr int EROWS = NB >= 32 ? NB / 32 : 1;
  constexpr int ECOLS = PCH * 4;
  constexpr int XGR = BM * 16;                      // 16-byte granules of an X chunk
  constexpr int BUF = XGR + NB * 8;                 // ... of a chunk buffer (X, then weights)
  constexpr int WS = D * BUF;                       // ... of a wave's ring
  constexpr int PCX = BM / 4, PCW = NB / 8;
  constexpr int PC = PCX + PCW;                     // loads per chunk
  static_assert(EROWS * PCH <= WAVE, "one exponent word (a chunk of a block row) per lane of wave 0");
  static_assert(D >= 1 && D <= CW && D * PC <= 63, "ring depth, counter range");
  __shared__ uint32_t e_words[WAVE];                // every lane of the load writes its word
  const uint8_t* const e_lds = reinterpret_cast<const uint8_t*>(e_words);
  __shared__ uint4 ring[NWK * WS];

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wk = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N;
  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // exponent words (one 4-byte word = the four K blocks of a chunk), EROWS block rows x the
  // workgroup's chunks, straight into LDS by wave 0 before its chunk loads (K is whole chunks, so
  // every word is aligned)
  if (wk == 0) {
    const int er = lane / PCH, cl = lane % PCH;
    const bool ok = lane < EROWS * PCH && c_begin + cl < c_end;
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32 + er) * KB + (c_begin + cl) * 4);
    lds_load4(re, lds_addr(e_words), ok ? off : OOB);
  }

  // This lane's share of a chunk's loads (the chunk index only adds c*128 to the offsets).
  //  X load i: rows 4i .. 4i+3; the lane fills row 4i + q4, slot r16 with granule r16 ^ (row % 16).
  uint32_t xoff[PCX];
  bool xok[PCX];
#pragma unroll
  for (int i = 0; i < PCX; ++i) {
    const int row = 4 * i + q4;
    const int m = m0 + row;
    xok[i] = m < M;
    xoff[i] = xok[i] ? (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + (r16 ^ (row & 15)) * 8) * 2) : 0u;
  }
  //  weight load i: rows 8i .. 8i+7; the lane fills row R = 8i + lane/8, slot lane%8 with granule
  //  (lane%8) ^ (R/2 % 8).
  uint32_t woff[PCW];
#pragma unroll
  for (int i = 0; i < PCW; ++i) {
    const int R = 8 * i + (lane >> 3);
    woff[i] = (uint32_t)(g * N + n0 + R) * (uint32_t)K + 16 * ((lane & 7) ^ ((R >> 1) & 7));
  }
  uint4* const area = ring + wk * WS;
  // chunk j of this wave is chunk c = c_begin + wk + j*NWK, into buffer j % D
  auto issue = [&](int j) {
    const int c = c_begin + wk + j * NWK;
    const bool cok = c < c_end;
    uint4* const b = area + (j % D) * BUF;
#pragma unroll
    for (int i = 0; i < PCX; ++i)
      lds_load16(rx, lds_addr(b + 64 * i), cok && xok[i] ? xoff[i] + (uint32_t)(c * KCH * 2) : OOB);
#pragma unroll
    for (int i = 0; i < PCW; ++i)
      lds_load16_stream(rq, lds_addr(b + XGR + 64 * i), cok ? woff[i] + (uint32_t)(c * KCH) : OOB);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) acc[mt][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wsw = (r16 >> 1) & 7;
  // A chunk's fragments (X, raw weight codes, block exponents) are read from its buffer first;
  // the buffer is then refilled at once and the dequant and MFMAs run from registers while the
  // next loads stream in.
  bf16x8_t xf[MT][4];
  uint4 wa[NT], wb[NT];
  uint32_t eb0[NT], eb1[NT];
  auto fetch = [&](int j) {
    const int cl = wk + j * NWK;                    // chunk index inside the workgroup
    const uint4* const b = area + (j % D) * BUF;
    // lane (r16, q4) takes the k values 64h + 16*q4 + 8u + [0, 8) of row r16 for MFMA 2h + u
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int gr = 8 * (f >> 1) + 2 * q4 + (f & 1);
        xf[mt][f] = __builtin_bit_cast(bf16x8_t, b[(mt * 16 + r16) * 16 + (gr ^ r16)]);
      }
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const int er = (n0 + ts * 16 + r16) / 32 - n0 / 32;
      eb0[ts] = e_lds[er * ECOLS + cl * 4 + (q4 >> 1)];
      eb1[ts] = e_lds[er * ECOLS + cl * 4 + 2 + (q4 >> 1)];
      wa[ts] = b[XGR + (ts * 16 + r16) * 8 + (q4 ^ wsw)];
      wb[ts] = b[XGR + (ts * 16 + r16) * 8 + ((4 + q4) ^ wsw)];
    }
  };
  auto math = [&]() {
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const float sc0 = block_scale(eb0[ts]);
      const float sc1 = block_scale(eb1[ts]);
      const bf16x8_t w0 = dequant8(wa[ts].x, wa[ts].y, sc0);
      const bf16x8_t w1 = dequant8(wa[ts].z, wa[ts].w, sc0);
      const bf16x8_t w2 = dequant8(wb[ts].x, wb[ts].y, sc1);
      const bf16x8_t w3 = dequant8(wb[ts].z, wb[ts].w, sc1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t c = acc[mt][ts];
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, xf[mt][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, xf[mt][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, xf[mt][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, xf[mt][3], c, 0, 0, 0);
        acc[mt][ts] = c;
      }
    }
  };

#pragma unroll
  for (int j = 0; j < D; ++j) issue(j);
  pin_epilogue_args(p);                             // the first loads are issued
  if (wk == 0) wait_vmcnt_le<D * PC>();             // wave 0's exponent words are in
  __syncthreads();
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    // this wave's loads of chunk j (those of the later chunks in flight may still be outstanding)
    if (j + D - 1 < CW) {
      wait_vmcnt_le<(D - 1) * PC>();
    } else {
      wait_vmcnt_le<0>();
    }
    const bool live = c_begin + wk + j * NWK < c_end;
    if (live) fetch(j);
    if (j + D < CW) {
      // this wave's reads of the buffer are done (the compiler sees the wait, so the MFMAs below
      // need none of their own)
      __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(j + D);
    }
    if (live) math();
  }
  wait_vmcnt_le<0>();                               // no load may still be writing LDS
  rows_epilogue<MT, NT, NWK, WS>(p, acc, reinterpret_cast<f32x4_t*>(ring), wk, lane, m0, n0, g, s);
}

// Tile kernel for many rows or wide weights: a BM x NB output tile per workgroup, BM = 16*MT*NWM
// rows of X and NB = 16*NT*NWN weight rows, NWM x NWN waves (each a 16*MT x 16*NT sub-tile), one
// 128-wide K chunk per step (K must be a multiple of 128).
//  * Both operands stream from memory straight into LDS with the buffer loads' LDS mode (no
//    VGPRs), through a ring of D stages: D - 1 chunks are in flight while one is computed. In a
//    stage, the X chunk is row-major (16 lanes fill one 256-byte row, each lane fetching the
//    granule that belongs in its slot), granule g of row r at slot g ^ (r % 16): the MFMA
//    fragment reads (16 rows x one granule per quarter wave) then run without LDS bank conflicts
//    (measured with the LDS bank-conflict counter; the XOR with r % 16 is one of the patterns that
//    measure conflict-free on gfx950). The weight chunk is read with eight lanes per
//    row (128 contiguous bytes per row and load: HBM streams this at about 6.7 TB/s on the
//    wide-weight shapes, the MFMA lane order - four lanes per row - at about 4.6) and stored
//    row-major, granule g of row R at slot g ^ (R/2 % 8), which spreads the fragment reads (16
//    rows x one granule) over 16 bank groups.
//  * The loads into LDS are not tracked by the compiler: each wave waits for its own loads of
//    chunk j with an explicit s_waitcnt on the vector memory counter (every wave issues the same
//    number of loads per chunk, out-of-range ones included), then one barrier per chunk makes the
//    stage visible to all waves and guarantees that every wave has finished chunk j - 1, whose
//    stage is refilled next.
//  * The exponent bytes of the workgroup's K range are staged once.
//  * With splits > 1 each workgroup stores its fp32 partial tile to the workspace [S][M][G][N]
//    and a second kernel sums the partials in ascending split order.
template <int MT, int NT, int NWM, int NWN, int D, int GI>
__global__ void __launch_bounds__(WAVE * NWM * NWN)
gemm_tile_kernel(KParams p) {
  constexpr int NWAVE = NWM * NWN;
  constexpr int BM = 16 * MT * NWM;
  constexpr int NB = 16 * NT * NWN;
  constexpr int XST = BM * 16;                      // 16-byte granules of an X stage
  constexpr int WST = NB * 8;                       // ... of a weight stage (NB rows x 128 bytes)
  constexpr int XI = BM / 4;                        // X loads per chunk (64 lanes = 4 rows)
  constexpr int WI = NB / 8;                        // weight loads per chunk (16 rows x 64 bytes)
  constexpr int PCX = XI / NWAVE, PCW = WI / NWAVE;
  constexpr int PC = PCX + PCW;                     // loads per wave per chunk
  constexpr int EROWS = NB / 32;
  constexpr int ESTR = TILE_MAX_CPS * 4;            // bytes per exponent row (64 lanes x 4)
  static_assert(XI % NWAVE == 0 && WI % NWAVE == 0, "every wave issues the same loads");
  static_assert(GI >= 1 && D >= GI + 1 && (D - 2) * PC <= 63, "ring depth, issue group, counter range");
  static_assert(NB % 32 == 0, "whole exponent block rows");
  __shared__ uint4 ring[D][XST + WST];
  __shared__ uint8_t e_lds[EROWS * ESTR];

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int nch = c_end - c_begin;
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // exponent bytes of the whole range, one 4-byte word (one chunk) per lane and block row,
  // loaded first (K is a multiple of 128, so every word is aligned)
  for (int er = wave; er < EROWS; er += NWAVE) {
    const int kb = (c_begin + lane) * 4;
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32 + er) * KB + kb);
    lds_load4(re, lds_addr(e_lds + er * ESTR), lane < nch && kb < KB ? off : OOB);
  }

  // This lane's share of the loads of a chunk (the chunk index only adds c*128 to the offsets).
  //  X load t: rows 4*i .. 4*i+3 (i = wave + t*NWAVE); the lane fills row 4i + q4, slot r16 with
  //  granule r16 ^ (row % 16) of that row.
  uint32_t xoff[PCX];
  bool xok[PCX];
#pragma unroll
  for (int u = 0; u < PCX; ++u) {
    const int i = wave + u * NWAVE;
    const int row = 4 * i + q4;
    const int gsrc = r16 ^ (row & 15);
    const int m = m0 + row;
    xok[u] = m < M;
    xoff[u] = xok[u] ? (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + gsrc * 8) * 2) : 0u;
  }
  //  weight load t: i = wave + t*NWAVE covers weight rows 8i .. 8i+7, eight lanes per row (128
  //  contiguous bytes per row: the DRAM-friendly width); the lane fills row R = 8i + lane/8, slot
  //  lane%8 with granule (lane%8) ^ ((R/2) % 8) of the row's chunk.
  uint32_t woff[PCW];
#pragma unroll
  for (int u = 0; u < PCW; ++u) {
    const int i = wave + u * NWAVE;
    const int row = 8 * i + (lane >> 3);
    const int gsrc = (lane & 7) ^ ((row >> 1) & 7);
    woff[u] = (uint32_t)(g * N + n0 + row) * (uint32_t)K + 16 * gsrc;
  }
  auto issue = [&](int j) {
    const int c = c_begin + j;
    const bool cok = c < c_end;
    const uint4* st = ring[j % D];
#pragma unroll
    for (int u = 0; u < PCX; ++u) {
      const int i = wave + u * NWAVE;
      lds_load16(rx, lds_addr(st + 4 * i * 16), cok && xok[u] ? xoff[u] + (uint32_t)(c * KCH * 2) : OOB);
    }
#pragma unroll
    for (int u = 0; u < PCW; ++u) {
      const int i = wave + u * NWAVE;
      lds_load16_stream(rq, lds_addr(st + XST + i * 64), cok ? woff[u] + (uint32_t)(c * KCH) : OOB);
    }
  };

#pragma unroll
  for (int j = 0; j < D - GI; ++j) issue(j);
  pin_epilogue_args(p);                             // the first loads are issued

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) acc[mt][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = r16;                               // slot swizzle of the X rows this lane reads
  const int wsw = (r16 >> 1) & 7;                   // ... and of its weight row
  // Chunks are issued in groups of GI (consecutive 128-byte pieces of each weight row arrive
  // back to back, which keeps DRAM pages open), at the first step of each group, into the GI
  // stages the previous group used. Before that issue D - 1 - GI chunks follow chunk j; at step r
  // of a group, D - 1 - r.
  auto step = [&](int j, auto rc) {
    constexpr int r = decltype(rc)::value;
    wait_vmcnt_le<(r == 0 ? D - 1 - GI : D - 1 - r) * PC>();   // this wave's loads of chunk j
    lds_barrier();                                  // ... everyone's; chunk j-1 is consumed
    if constexpr (r == 0) {
#pragma unroll
      for (int t = 0; t < GI; ++t) issue(j + D - GI + t);
    }
    if (j >= nch) return;                           // padding step of the last group
    const uint4* st = ring[j % D];
    bf16x8_t xf[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* xrow = st + (wm * 16 * MT + mt * 16 + r16) * 16;
      xf[mt][0] = __builtin_bit_cast(bf16x8_t, xrow[(2 * q4) ^ fr]);
      xf[mt][1] = __builtin_bit_cast(bf16x8_t, xrow[(2 * q4 + 1) ^ fr]);
      xf[mt][2] = __builtin_bit_cast(bf16x8_t, xrow[(8 + 2 * q4) ^ fr]);
      xf[mt][3] = __builtin_bit_cast(bf16x8_t, xrow[(9 + 2 * q4) ^ fr]);
    }
    const int e0 = j * 4 + (q4 >> 1);
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const int tile = wn * NT + ts;
      const uint4* wrow = st + XST + (16 * tile + r16) * 8;
      const uint4 a = wrow[q4 ^ wsw];
      const uint4 b = wrow[(4 + q4) ^ wsw];
      const int er = (16 * tile + r16) >> 5;
      const float sc0 = block_scale(e_lds[er * ESTR + e0]);
      const float sc1 = block_scale(e_lds[er * ESTR + e0 + 2]);
      const bf16x8_t w0 = dequant8(a.x, a.y, sc0);
      const bf16x8_t w1 = dequant8(a.z, a.w, sc0);
      const bf16x8_t w2 = dequant8(b.x, b.y, sc1);
      const bf16x8_t w3 = dequant8(b.z, b.w, sc1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t c = acc[mt][ts];
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, xf[mt][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, xf[mt][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, xf[mt][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, xf[mt][3], c, 0, 0, 0);
        acc[mt][ts] = c;
      }
    }
  };
  for (int j0 = 0; j0 < nch; j0 += GI) {
    step(j0, std::integral_constant<int, 0>{});
    if constexpr (GI > 1) step(j0 + 1, std::integral_constant<int, 1 % GI>{});
    if constexpr (GI > 2) step(j0 + 2, std::integral_constant<int, 2 % GI>{});
    if constexpr (GI > 3) step(j0 + 3, std::integral_constant<int, 3 % GI>{});
  }
  wait_vmcnt_le<0>();                               // no load may still be writing LDS at exit

  // MXFP8 output (one split): the wave's sub-tile holds whole 32-column blocks (tiles 2b, 2b+1)
  if (p.yq) {
    if constexpr (NT % 2 == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + wm * 16 * MT + mt * 16 + r16;
#pragma unroll
        for (int bk = 0; bk < NT / 2; ++bk) {
          uint32_t c_lo, c_hi;
          const uint8_t sb = mx_block_codes(acc[mt][2 * bk], acc[mt][2 * bk + 1], c_lo, c_hi);
          if (m < M) store_mx_block(p.yq, p.ys, m, g, G, N, n0 + wn * 16 * NT + 32 * bk, q4, c_lo, c_hi, sb);
        }
      }
    }
    return;
  }

  // output: this wave's sub-tile, or its fp32 partial for the reduce kernel
  float* const part = reinterpret_cast<float*>(p.slots);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + wm * 16 * MT + mt * 16 + r16;
    if (m >= M) continue;
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const size_t o = ((size_t)m * G + g) * N + n0 + wn * 16 * NT + ts * 16 + q4 * 4;
      const f32x4_t v = acc[mt][ts];
      if (p.splits > 1) {
        *reinterpret_cast<f32x4_t*>(part + (size_t)s * M * G * N + o) = v;
      } else if (p.out_f32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = v;
      } else {
        const uint2 w2 = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
      }
    }
  }
}

// Decode kernel (at most XR rows of X per workgroup, one pass over its K range; K a multiple of
// 128). The weight is the A operand as everywhere; what differs is how the bytes arrive: all of
// them stream into LDS with the buffer loads' LDS mode, so the loads are issued at once and cost
// no VGPRs:
//  * the exponent words of the workgroup's range (one 4-byte word = one chunk of a block row);
//  * the workgroup's X rows, dense, one granule of padding per row (fragment reads of 16 lanes
//    then hit 16 distinct bank groups);
//  * each wave's weight chunks, eight lanes per weight row: 128 contiguous bytes per row and
//    load, which HBM streams far better than the MFMA order (64 bytes per row), stored row-major
//    with granule g of row R at slot g ^ (R/2 % 8) (conflict-free fragment reads).
// Each wave counts its own loads: it waits for its exponent and X loads and meets the others at
// a barrier (X is shared), then computes each of its chunks as soon as that chunk's weight pieces
// have landed. Out-of-range weight loads are issued too (so that every wave's count of them is
// fixed), but what they leave in LDS is never used: chunks past the range are skipped, and X rows
// at or beyond M (not loaded at all) feed only output columns that are not stored. Waves along K
// are summed through LDS in ascending order, as in the other one-pass kernels, so an output's fp32
// sum is the same chain of chunks as in gemm_direct_kernel with the same NWK and chunks per split.
// RG = true takes K that is not a multiple of 128: the last chunk's X, weight and exponent
// reads past K return zeros (exponent factors there are 1), so the fp32 chains are those of K
// zero-padded to whole chunks; the aligned instances carry none of these checks.
// RS = 1 takes one exponent byte per weight row and 32 columns (e [G][N][K/32]; page
// "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row draft_main_proj) instead of one per
// 32x32 block: the exponent words are then staged per weight row, nothing else changes.
// TR = real weight rows per 16-row MFMA tile: with TR = 8 a workgroup holds half as many weight
// rows, so a long K range still fits its LDS in one pass; the MFMA's rows 8..15 then repeat rows
// 0..7 and their outputs are not stored.
// XGP > 0 (G = 8 / XGP groups): the workgroups of group g run on XCDs XGP*g .. XGP*g + XGP - 1 (the
// hardware deals workgroups to the 8 XCDs by linear index mod 8), so each XCD's L2 fetches the
// activation rows of one group instead of all of them.
template <int NT, int NWN, int NWK, int CW, int XR, int RS, int TR, bool RG = false, int XGP = 0>
__global__ void __launch_bounds__(WAVE * NWN * NWK)
gemm_decode_kernel(KParams p) {
  static_assert(XGP == 0 || XGP == 2 || XGP == 4, "XCDs per group");
  constexpr int NWAVE = NWN * NWK;
  constexpr int NB = TR * NT * NWN;
  constexpr int TG = TR * 8;                        // granules of one tile's chunk in LDS
  constexpr int PCH = NWK * CW;                     // chunks of the workgroup
  constexpr int ROWG = PCH * 16 + 1;                // granules per LDS X row (one of padding)
  constexpr int XI = XR * PCH / 4;                  // X loads: 1 KB = 4 chunks of one row
  constexpr int XPW = XI / NWAVE;
  constexpr int WPW = CW * NT * (TR / 8);           // weight loads per wave
  constexpr int EROWS = RS ? NB : (NB >= 32 ? NB / 32 : 1);   // exponent rows staged
  static_assert(XI % NWAVE == 0 && XPW >= 1, "every wave issues the same X loads");
  static_assert(PCH <= 64, "one exponent word per lane and chunk");
  static_assert(!RG || (RS == 0 && PCH * 4 + 3 <= 256), "ragged K: block exponents, a shifted row in one load");
  static_assert((XR & (XR - 1)) == 0 && XR <= 16, "X rows: a power of two up to 16");
  static_assert(XPW + WPW + 1 <= 63, "vector memory counter range");
  static_assert(TR == 8 || TR == 16, "tile rows");
  __shared__ uint4 x_lds[XR * ROWG];
  __shared__ uint4 w_lds[NWAVE * CW * NT * TG];
  __shared__ uint32_t e_lds[EROWS * 64];
  __shared__ f32x4_t red[NWK > 1 ? (NWK - 1) * NWN * NT * WAVE : 1];

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wk = wave / NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  Tile tl = tile_of_grid(p);
  if constexpr (XGP > 0) {
    // linear index L = x + y * nblocks over nblocks x G workgroups: XCD L % 8, slot L / 8
    const int L = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
    tl.g = (L & 7) / XGP;
    tl.nb = (L & (XGP - 1)) + (L >> 3) * XGP;
  }
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * NB, m0 = mb * XR;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // (1) exponent words: wave w loads exponent rows w, w + NWAVE, ... (block rows, or weight rows
  //     with RS), lane l the word of chunk c_begin + l. The count may differ between waves: these
  //     loads come first, and the waits below count only the weight loads issued after them.
  //     RG (K not a multiple of 128): a row's bytes need not start on a word; the words are
  //     loaded from the aligned address below the range's first byte, and the reads add that
  //     offset.
  for (int er = wave; er < EROWS; er += NWAVE) {
    const int c = c_begin + lane;
    const int erow = RS ? g * N + n0 + er : g * (N / 32) + n0 / 32 + er;
    if constexpr (RG) {
      const uint32_t first = (uint32_t)(erow * KB + c_begin * 4);
      const uint32_t end = (uint32_t)(erow * KB + min(c_end * 4, KB));
      const uint32_t wd = (first & ~3u) + 4u * (uint32_t)lane;
      lds_load4(re, lds_addr(e_lds + er * 64), wd < end ? wd : OOB);
    } else {
      const uint32_t off = (uint32_t)(erow * KB + c * 4);
      lds_load4(re, lds_addr(e_lds + er * 64), c < c_end ? off : OOB);
    }
  }
  // (2) X rows m0 .. m0+XR-1 over the workgroup's chunks: load i covers row i / (PCH/4), granules
  //     64*(i % (PCH/4)) .. +63 of the row's range. Rows at or beyond M are not loaded (the waits
  //     below count only the weight loads issued after these, so the number may vary).
#pragma unroll
  for (int u = 0; u < XPW; ++u) {
    const int i = wave + u * NWAVE;
    const int row = i / (PCH / 4), pc = i % (PCH / 4);
    const int m = m0 + row;
    const int k = c_begin * KCH + (pc * 64 + lane) * 8;
    const uint32_t off = (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + k) * 2);
    const bool ok = k < c_end * KCH && (!RG || k < K);   // RG: values past K read zeros
    if (m < M) lds_load16(rx, lds_addr(x_lds + row * ROWG + pc * 64), ok ? off : OOB);
  }
  // (3) this wave's weight chunks: load (j, ts, v) covers rows 8v .. 8v+7 of its tile ts (TR
  //     rows), the lane fills row R = 8v + lane/8, slot lane%8 with granule (lane%8) ^ (R/2 % 8)
  uint4* const wbase = w_lds + wave * CW * NT * TG;
  {
    const int R0 = lane >> 3;
    const uint32_t qrow = (uint32_t)(g * N + n0 + wn * TR * NT + R0) * (uint32_t)K;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int c = c_begin + wk + j * NWK;
#pragma unroll
      for (int ts = 0; ts < NT; ++ts)
#pragma unroll
        for (int v = 0; v < TR / 8; ++v) {
          const int R = 8 * v + R0;
          const int gsrc = (lane & 7) ^ ((R >> 1) & 7);
          const uint32_t off = qrow + (uint32_t)((ts * TR + 8 * v) * K + c * KCH + gsrc * 16);
          const bool ok = c < c_end && (!RG || c * KCH + gsrc * 16 < K);   // RG: codes past K read zeros
          lds_load16_stream(rq, lds_addr(wbase + (j * NT + ts) * TG + v * 64), ok ? off : OOB);
        }
    }
  }
  pin_epilogue_args(p);                             // every load is issued
  wait_vmcnt_le<WPW>();                             // this wave's exponent and X loads
  lds_barrier();                                    // ... everyone's

  // (4) X fragments and block factors of all this wave's chunks into registers (X and the
  //     exponents are complete since the barrier), so that each chunk, once its own weights have
  //     landed, costs one LDS round trip (its weight fragments) before its dequant + MFMAs. Chunks
  //     are computed in ascending order.
  f32x4_t acc[NT];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts) acc[ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4* xrow = x_lds + (r16 & (XR - 1)) * ROWG;   // rows beyond XR feed unused columns
  const uint8_t* eb = reinterpret_cast<const uint8_t*>(e_lds);
  const int wr = r16 & (TR - 1);                   // the weight row this lane reads (rows TR..15
  const int wsw = (wr >> 1) & 7;                    // of a half tile repeat rows 0..7)
  bf16x8_t xf[CW][4];
  float sc[CW][NT][2];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int cl = wk + j * NWK;                    // chunk index inside the workgroup
    xf[j][0] = __builtin_bit_cast(bf16x8_t, xrow[cl * 16 + 2 * q4]);
    xf[j][1] = __builtin_bit_cast(bf16x8_t, xrow[cl * 16 + 2 * q4 + 1]);
    xf[j][2] = __builtin_bit_cast(bf16x8_t, xrow[cl * 16 + 8 + 2 * q4]);
    xf[j][3] = __builtin_bit_cast(bf16x8_t, xrow[cl * 16 + 9 + 2 * q4]);
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const int er = RS ? wn * TR * NT + ts * TR + wr : (n0 + wn * TR * NT + ts * TR + wr) / 32 - n0 / 32;
      if constexpr (RG) {
        const int erow = g * (N / 32) + n0 / 32 + er;
        const int sh = (erow * KB + c_begin * 4) & 3;  // the range's first byte within its word
        const int kb = (c_begin + cl) * 4 + (q4 >> 1);  // this lane's first block of the chunk
        // blocks past K (their codes read as zeros) take a unit factor, never a stray byte
        sc[j][ts][0] = kb < KB ? block_scale(eb[er * 256 + sh + cl * 4 + (q4 >> 1)]) : 1.0f;
        sc[j][ts][1] = kb + 2 < KB ? block_scale(eb[er * 256 + sh + cl * 4 + 2 + (q4 >> 1)]) : 1.0f;
      } else {
        sc[j][ts][0] = block_scale(eb[er * 256 + cl * 4 + (q4 >> 1)]);
        sc[j][ts][1] = block_scale(eb[er * 256 + cl * 4 + 2 + (q4 >> 1)]);
      }
    }
  }
  auto chunk = [&](int j) {
    const int cl = wk + j * NWK;
    // (a chunk past the range was not loaded: its LDS holds nothing defined)
    if (c_begin + cl >= c_end) return;
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) {
      const uint4* wt = wbase + (j * NT + ts) * TG + wr * 8;
      const uint4 a = wt[q4 ^ wsw], b = wt[(4 + q4) ^ wsw];
      f32x4_t c = acc[ts];
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.x, a.y, sc[j][ts][0]), xf[j][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.z, a.w, sc[j][ts][0]), xf[j][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.x, b.y, sc[j][ts][1]), xf[j][2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.z, b.w, sc[j][ts][1]), xf[j][3], c, 0, 0, 0);
      acc[ts] = c;
    }
  };
  constexpr int WPC = NT * (TR / 8);                // weight loads per chunk
  wait_vmcnt_le<(CW - 1) * WPC>();
  chunk(0);
  if constexpr (CW > 1) { wait_vmcnt_le<(CW - 2 >= 0 ? CW - 2 : 0) * WPC>(); chunk(1); }
  if constexpr (CW > 2) { wait_vmcnt_le<(CW - 3 >= 0 ? CW - 3 : 0) * WPC>(); chunk(2); }
  if constexpr (CW > 3) { wait_vmcnt_le<(CW - 4 >= 0 ? CW - 4 : 0) * WPC>(); chunk(3); }
  if constexpr (CW > 4) { wait_vmcnt_le<(CW - 5 >= 0 ? CW - 5 : 0) * WPC>(); chunk(4); }
  if constexpr (CW > 5) { wait_vmcnt_le<(CW - 6 >= 0 ? CW - 6 : 0) * WPC>(); chunk(5); }
  if constexpr (CW > 6) { wait_vmcnt_le<(CW - 7 >= 0 ? CW - 7 : 0) * WPC>(); chunk(6); }
  if constexpr (CW > 7) { wait_vmcnt_le<(CW - 8 >= 0 ? CW - 8 : 0) * WPC>(); chunk(7); }
  static_assert(CW <= 8, "chunks per wave");

  // (5) waves along K: ascending-order sum through LDS
  if constexpr (NWK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) red[(((wk - 1) * NWN + wn) * NT + ts) * WAVE + lane] = acc[ts];
    }
    __syncthreads();
    if (wk != 0) return;
    f32x4_t part[NWK - 1][NT];                      // all reads issued before the first add
#pragma unroll
    for (int w = 1; w < NWK; ++w)
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) part[w - 1][ts] = red[(((w - 1) * NWN + wn) * NT + ts) * WAVE + lane];
#pragma unroll
    for (int w = 1; w < NWK; ++w)
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) acc[ts] += part[w - 1][ts];
  }
  // (6) output
  const int m = m0 + r16;
  const bool mrow = r16 < XR && m < M && q4 * 4 < TR;   // a real X row and a real weight row
  if (p.splits == 1) {
    if (mrow) {
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int n = n0 + wn * TR * NT + ts * TR + q4 * 4;
        const size_t o = ((size_t)m * G + g) * N + n;
        const f32x4_t v = acc[ts];
        if (p.out_f32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = v;
        } else {
          const uint2 w2 = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
        }
      }
    }
    return;
  }
  constexpr int NV = NT * 4;
  float v[NV];
  size_t off[NV];
  int mr[NV];
  bool live[NV];
#pragma unroll
  for (int ts = 0; ts < NT; ++ts)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[ts * 4 + r] = acc[ts][r];
      off[ts * 4 + r] = ((size_t)m * G + g) * N + n0 + wn * TR * NT + ts * TR + q4 * 4 + r;
      mr[ts * 4 + r] = m;
      live[ts * 4 + r] = mrow;
    }
  combine_splits<NV>(p, s, v, off, mr, live);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (live[i]) store_out(p, off[i], v[i]);
}

// Slab kernel for mid row counts on narrow weights: a BM x NB output tile per workgroup over its
// whole K range, the X slab shared by all waves through LDS. What bounds these shapes is the rate
// at which one CU can pull L2-resident data: a wave load that reads one contiguous kilobyte runs
// at about 100 GB/s per CU, one spread over two to sixteen rows (the fragment-friendly shapes) at
// about 60. So the K range is walked in slabs of four chunks (512 values, one kilobyte of each X
// row), and every X load fetches one whole row piece:
//  * a stage of the LDS ring holds the X slab (BM rows x 1 KB, row-major, granule g of row r at
//    slot g ^ (r % 16), so that the fragment reads of 16 rows at one k hit 16 distinct bank groups)
//    and the weight slab (NB rows x 512 bytes, two rows per load, granule g of row R at slot
//    g ^ (R % 16)); each lane fetches the granule that belongs in its slot, so a load still covers
//    exactly one contiguous kilobyte (X) or two 512-byte row pieces (weights);
//  * S - 1 slabs are in flight while one is computed; each wave counts its own loads (every wave
//    issues the same number per slab) and one barrier per slab publishes the stage and frees the
//    one consumed before;
//  * NWM x NWN x NWK waves: a wave owns a 16*MT x 16*NT sub-tile and the chunks
//    wk*CPW .. wk*CPW + CPW - 1 of every slab (CPW = 4 / NWK), so each output's fp32 sum is
//    NWK ascending chains, which are added through LDS in ascending wk order at the end;
//  * with more than one split (whole slabs per split) the partials meet in the pairwise-exchange
//    tree of the one-pass kernels.
constexpr int SLAB_CH = 4;                          // chunks per slab

template <int MT, int NT, int NWM, int NWN, int NWK, int S>
__global__ void __launch_bounds__(WAVE * NWM * NWN * NWK)
gemm_slab_kernel(KParams p) {
  constexpr int NWAVE = NWM * NWN * NWK;
  constexpr int BM = 16 * MT * NWM;
  constexpr int NB = 16 * NT * NWN;
  constexpr int CPW = SLAB_CH / NWK;                // chunks of a slab per wave
  constexpr int XG = BM * 64;                       // 16-byte granules of an X slab
  constexpr int WGR = NB * 32;                      // ... of a weight slab
  constexpr int PCX = BM / NWAVE, PCW = NB / 2 / NWAVE;
  constexpr int PC = PCX + PCW;                     // loads per wave per slab
  constexpr int EROWS = NB / 32;
  constexpr int ESTR = TILE_MAX_CPS * 4;
  constexpr int TILES = MT * NT;
  static_assert(SLAB_CH % NWK == 0, "waves along K split a slab evenly");
  static_assert(BM % NWAVE == 0 && (NB / 2) % NWAVE == 0, "every wave issues the same loads");
  static_assert(S >= 2 && (S - 2) * PC <= 63, "ring depth, counter range");
  static_assert(NB % 32 == 0, "whole exponent block rows");
  static_assert((NWK - 1) * NWM * NWN * TILES * WAVE * 16 <= S * (XG + WGR) * 16, "reduction fits the ring");
  // MXFP8 output in the kernel: whole 32-column blocks, every wave's partial tiles in the ring
  constexpr bool MX_OK = NB % 32 == 0 && NWK * NWM * NWN * TILES * WAVE * 16 <= S * (XG + WGR) * 16;
  __shared__ uint4 ring[S][XG + WGR];
  __shared__ uint8_t e_lds[EROWS * ESTR];

  prefetch_args(p);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wk = wave / (NWM * NWN), wmn = wave % (NWM * NWN);
  const int wm = wmn / NWN, wn = wmn % NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  const Tile tl = tile_of(p);
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;                    // a multiple of SLAB_CH
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int nch = c_end - c_begin;
  const int nslab = (nch + SLAB_CH - 1) / SLAB_CH;
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);

  // exponent words of the split's range (one 4-byte word = one chunk of a block row)
  for (int er = wave; er < EROWS; er += NWAVE) {
    const int kb = (c_begin + lane) * 4;
    const uint32_t off = (uint32_t)((g * (N / 32) + n0 / 32 + er) * KB + kb);
    lds_load4(re, lds_addr(e_lds + er * ESTR), lane < nch && kb < KB ? off : OOB);
  }

  // X load u: tile row i = wave + u*NWAVE, the lane fetches granule lane ^ (i % 16) of the row's
  // kilobyte. Weight load u: rows 2i, 2i + 1 (i = wave + u*NWAVE), the lane fetches granule
  // (lane % 32) ^ (R % 16) of row R = 2i + lane/32.
  uint32_t xoff[PCX];
  bool xok[PCX];
#pragma unroll
  for (int u = 0; u < PCX; ++u) {
    const int i = wave + u * NWAVE;
    const int m = m0 + i;
    xok[u] = m < M;
    xoff[u] = xok[u] ? (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + (lane ^ (i & 15)) * 8) * 2) : 0u;
  }
  uint32_t woff[PCW];
#pragma unroll
  for (int u = 0; u < PCW; ++u) {
    const int i = wave + u * NWAVE;
    const int R = 2 * i + (lane >> 5);
    woff[u] = (uint32_t)(g * N + n0 + R) * (uint32_t)K + 16 * ((lane & 31) ^ (R & 15));
  }
  auto issue = [&](int j) {
    const int c0 = c_begin + j * SLAB_CH;           // first chunk of slab j
    const bool sok = j < nslab;
    const uint4* st = ring[j % S];
#pragma unroll
    for (int u = 0; u < PCX; ++u) {
      const int i = wave + u * NWAVE;
      const uint32_t k2 = (uint32_t)(c0 * KCH * 2);
      lds_load16(rx, lds_addr(st + i * 64), sok && xok[u] && c0 * KCH + 8 * lane < K ? xoff[u] + k2 : OOB);
    }
#pragma unroll
    for (int u = 0; u < PCW; ++u) {
      const int i = wave + u * NWAVE;
      lds_load16_stream(rq, lds_addr(st + XG + i * 64), sok ? woff[u] + (uint32_t)(c0 * KCH) : OOB);
    }
  };

#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(j);
  pin_epilogue_args(p);                             // the first loads are issued

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts) acc[mt][ts] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < nslab; ++j) {
    wait_vmcnt_le<(S - 2) * PC>();                  // this wave's loads of slab j
    lds_barrier();                                  // ... everyone's; slab j - 1 is consumed
    issue(j + S - 1);
    const uint4* st = ring[j % S];
#pragma unroll
    for (int cc = wk * CPW; cc < wk * CPW + CPW; ++cc) {
      const int cl = j * SLAB_CH + cc;              // chunk index inside the split
      if (cl >= nch) break;
      bf16x8_t xf[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4* xrow = st + (wm * 16 * MT + mt * 16 + r16) * 64;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          xf[mt][u] = __builtin_bit_cast(bf16x8_t, xrow[(cc * 16 + 2 * q4 + (u & 1) + 8 * (u >> 1)) ^ r16]);
      }
      const int e0 = cl * 4 + (q4 >> 1);
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const int R = wn * 16 * NT + ts * 16 + r16;
        const uint4* wrow = st + XG + R * 32;
        const uint4 a = wrow[(cc * 8 + q4) ^ r16];
        const uint4 b = wrow[(cc * 8 + 4 + q4) ^ r16];
        const int er = R >> 5;
        const float sc0 = block_scale(e_lds[er * ESTR + e0]);
        const float sc1 = block_scale(e_lds[er * ESTR + e0 + 2]);
        const bf16x8_t w0 = dequant8(a.x, a.y, sc0);
        const bf16x8_t w1 = dequant8(a.z, a.w, sc0);
        const bf16x8_t w2 = dequant8(b.x, b.y, sc1);
        const bf16x8_t w3 = dequant8(b.z, b.w, sc1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t c = acc[mt][ts];
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, xf[mt][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, xf[mt][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, xf[mt][2], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, xf[mt][3], c, 0, 0, 0);
          acc[mt][ts] = c;
        }
      }
    }
  }
  wait_vmcnt_le<0>();                               // no load may still be writing LDS

  // MXFP8 output (one split): every wave parks its tiles in the ring; each job (a 16-row strip
  // and a 32-column block) adds the waves' tiles of its two 16-column halves in ascending wave
  // order - the sums of the bf16/fp32 path below - and quantises the block
  if (p.yq) {
    if constexpr (MX_OK) {
      lds_barrier();                                // every wave is done with the ring
      f32x4_t* red = reinterpret_cast<f32x4_t*>(&ring[0][0]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ts = 0; ts < NT; ++ts)
          red[((wk * NWM * NWN + wmn) * TILES + mt * NT + ts) * WAVE + lane] = acc[mt][ts];
      __syncthreads();
      constexpr int NBLK = NB / 32;
      constexpr int JOBS = NWM * MT * NBLK;
      for (int j = wave; j < JOBS; j += NWAVE) {
        const int jm = j / (MT * NBLK), mt = (j / NBLK) % MT, bk = j % NBLK;
        f32x4_t half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c16 = 32 * bk + 16 * h;         // first column of the half in the tile
          const int base = (jm * NWN + c16 / (16 * NT)) * TILES + mt * NT + (c16 / 16) % NT;
          f32x4_t v = red[base * WAVE + lane];
#pragma unroll
          for (int w = 1; w < NWK; ++w) v += red[(w * NWM * NWN * TILES + base) * WAVE + lane];
          half[h] = v;
        }
        uint32_t c_lo, c_hi;
        const uint8_t sb = mx_block_codes(half[0], half[1], c_lo, c_hi);
        const int m = m0 + jm * 16 * MT + mt * 16 + r16;
        if (m < M) store_mx_block(p.yq, p.ys, m, g, G, N, n0 + 32 * bk, q4, c_lo, c_hi, sb);
      }
    }
    return;
  }

  // waves along K: ascending-order sum through LDS (aliasing the ring)
  if constexpr (NWK > 1) {
    lds_barrier();                                  // every wave is done with the ring
    f32x4_t* red = reinterpret_cast<f32x4_t*>(&ring[0][0]);
    if (wk > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ts = 0; ts < NT; ++ts)
          red[(((wk - 1) * NWM * NWN + wmn) * TILES + mt * NT + ts) * WAVE + lane] = acc[mt][ts];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int w = 1; w < NWK; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ts = 0; ts < NT; ++ts)
          acc[mt][ts] += red[(((w - 1) * NWM * NWN + wmn) * TILES + mt * NT + ts) * WAVE + lane];
  }

  if (p.splits == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + wm * 16 * MT + mt * 16 + r16;
      if (m >= M) continue;
#pragma unroll
      for (int ts = 0; ts < NT; ++ts) {
        const size_t o = ((size_t)m * G + g) * N + n0 + wn * 16 * NT + ts * 16 + q4 * 4;
        const f32x4_t v = acc[mt][ts];
        if (p.out_f32) {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = v;
        } else {
          const uint2 w2 = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
        }
      }
    }
    return;
  }
  constexpr int NV = TILES * 4;
  float v[NV];
  size_t off[NV];
  int mr[NV];
  bool live[NV];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ts = 0; ts < NT; ++ts)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (mt * NT + ts) * 4 + r;
        const int m = m0 + wm * 16 * MT + mt * 16 + r16;
        v[i] = acc[mt][ts][r];
        off[i] = ((size_t)m * G + g) * N + n0 + wn * 16 * NT + ts * 16 + q4 * 4 + r;
        mr[i] = m;
        live[i] = m < M;
      }
  combine_splits<NV>(p, s, v, off, mr, live);
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (live[i]) store_out(p, off[i], v[i]);
}

// Paired decode kernel: at most 8 rows of X and 8 weight rows per workgroup, one pass over its K
// range, and each MFMA computing two chunks at once. In v_mfma_f32_16x16x32_bf16 the A rows
// 0..7 carry the workgroup's 8 weight rows at the first chunk of a pair and A rows 8..15 the same
// weight rows at the second chunk; the B columns 0..7 carry the X rows at the first chunk and
// columns 8..15 at the second. The diagonal 8 x 8 blocks of D are the two chunks' products (the
// off-diagonal ones mix chunks and are discarded) and a lane exchange adds them at the end. So
// every lane dequantises codes nobody else needs, and a workgroup of 8 weight rows costs half the
// dequant and MFMA work of a 16-row tile: the decode shapes then spread over twice as many
// workgroups (256 at wo_a, one per CU) at the same work per code.
//  * Wave wk owns the CW = 2 * CP consecutive chunks cw0 .. cw0 + CW - 1 of the workgroup's range
//    (pairs (cw0, cw0 + 1), (cw0 + 2, cw0 + 3), ...), and loads everything it reads itself, into
//    its own LDS: no barrier until the waves' sums meet.
//  * X: each row's CW * 256 bytes are contiguous (one kilobyte per row and load at CW = 4), read
//    with the LDS mode of the buffer loads; within each chunk's 16 granules of a row the granules
//    are rotated by (row + 8 * (chunk & 1)), which makes the fragment reads of the 16 lanes of a
//    quarter wave (8 rows x 2 chunks) hit 16 distinct bank groups.
//  * Weights: one load per chunk, eight lanes per row (128 contiguous bytes per row and load),
//    granule g of row R at slot g ^ (R / 2); chunk tiles 68 granules apart so that the two chunks
//    of a pair sit 4 granules apart in bank space (conflict-free fragment reads of both halves).
//  * Exponents: the wave's words of its block row (8 weight rows lie in one 32-row block).
//  * Chunks past the range (a split's end, or K in the last pair) are loaded as out-of-range
//    reads, which leave zeros, and take a unit factor.
// Each output's fp32 sum: per wave, the chain of the first chunks of its pairs and the chain of
// the second chunks, added; then the waves in ascending order. It depends on the chunk count, not
// on K, so K zero-padded inside the same chunk count gives the same sums.
// FULL instances serve the plans whose one split covers exactly the workgroup's NWK * CW chunks
// (K = 128 * NWK * CW): every chunk is then in range and no load, factor or output needs a range
// test, which shortens the path from the arguments to the first loads (each instruction there
// delays the whole stream) and the epilogue. Their sums are those of the general instance.
// WF weight chunks (at most two, the first pair's) are issued before the X rows, the rest after.
// XG (two groups, one m-block, one split): the workgroups of group 0 run on XCDs 0..3 and those of
// group 1 on XCDs 4..7 (the hardware deals workgroups to the 8 XCDs by linear index mod 8), so each
// XCD's L2 fetches the activation rows of one group instead of both.
template <int NWK, int CP, bool RG, bool FULL = false, int WF = 0, bool XG = false>
__global__ void __launch_bounds__(WAVE * NWK)
gemm_pair_kernel(KParams p) {
  static_assert(WF >= 0 && WF <= 2, "only the first pair's weight chunks go before the X rows");
  static_assert(!XG || FULL, "XCD grouping: the whole-range instances (one split)");
  constexpr int CW = 2 * CP;                        // chunks per wave
  constexpr int XR = 8;                             // rows of X per workgroup
  constexpr int XS = CW * 16;                       // granules of one X row slice
  constexpr int WT = 68;                            // granules per weight chunk tile (64 + offset)
  constexpr int XL = XR * XS / 64;                  // X loads per wave
  static_assert(CP == 1 || CP == 2 || CP == 4, "X row slices tile a wave load");
  static_assert(!RG || CW + 1 <= 64, "exponent words of a ragged range");
  static_assert(!(RG && FULL), "a whole range has no ragged chunk");
  __shared__ uint4 x_lds[NWK * XR * XS];
  __shared__ uint4 w_lds[NWK * CW * WT];
  __shared__ uint32_t e_lds[NWK * 64];
  __shared__ f32x4_t red[NWK > 1 ? (NWK - 1) * 16 : 1];

  prefetch_args(p);
  const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;

  Tile tl = tile_of_grid(p);
  if constexpr (XG) {
    // linear index L = x + y * nblocks over nblocks x 2 workgroups: XCD L % 8, slot L / 8
    const int L = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
    tl.g = (L & 7) >> 2;
    tl.nb = (L & 3) + ((L >> 3) << 2);
  }
  const int mb = tl.mb, nb = tl.nb, g = tl.g, s = tl.s;

  const int K = p.K, M = p.M, N = p.N, G = p.G;
  const int n0 = nb * 8, m0 = mb * XR;
  const int c_begin = FULL ? 0 : s * p.cps;
  const int c_end = FULL ? NWK * CW : min(c_begin + p.cps, p.kchunks);
  const int cw0 = c_begin + wk * CW;                // this wave's first chunk
  const int KB = K / 32;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, (int)p.x_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, 0, (int)p.q_bytes, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc((void*)p.e, 0, (int)p.e_bytes, RSRC_WORD3);
  uint4* const xw = x_lds + wk * XR * XS;
  uint4* const ww = w_lds + wk * CW * WT;
  uint32_t* const ew = e_lds + wk * 64;
  const int erow = g * (N / 32) + n0 / 32;

  // (1) exponent words of the wave's chunks (RG: from the aligned word below the first byte)
  if constexpr (RG) {
    const uint32_t first = (uint32_t)(erow * KB + cw0 * 4);
    const uint32_t end = (uint32_t)(erow * KB + min(min(cw0 + CW, c_end) * 4, KB));
    const uint32_t wd = (first & ~3u) + 4u * (uint32_t)lane;
    lds_load4(re, lds_addr(ew), lane <= CW && wd < end ? wd : OOB);
  } else {
    const int c = cw0 + lane;
    lds_load4(re, lds_addr(ew), lane < CW && (FULL || c < c_end) ? (uint32_t)(erow * KB + c * 4) : OOB);
  }
  // (3) weight chunks, one load each: lane l fills row R = l / 8, slot l % 8 with granule
  //     (l % 8) ^ (R / 2); the first WF of them before the X rows
  const int wR = lane >> 3;
  const int wgsrc = (lane & 7) ^ (wR >> 1);
  const uint32_t qrow = (uint32_t)(g * N + n0 + wR) * (uint32_t)K;
  auto wload = [&](int cl) {
    const int c = cw0 + cl;
    const uint32_t off = qrow + (uint32_t)(c * KCH + wgsrc * 16);
    const bool ok = (FULL || c < c_end) && (!RG || c * KCH + wgsrc * 16 < K);
    lds_load16_stream(rq, lds_addr(ww + cl * WT), ok ? off : OOB);
  };
#pragma unroll
  for (int cl = 0; cl < WF; ++cl) wload(cl);
  // (2) X rows m0 .. m0 + 7 over the wave's chunks: load i fills slots 64i .. 64i + 63 of the rows'
  //     slices (row-major); the lane fetches the granule that belongs in its slot. Loads whose rows
  //     all lie at or beyond M are skipped (those rows feed only discarded columns).
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int pos = i * 64 + lane;
    const int row = pos / XS, slot = pos % XS;
    const int cl = slot / 16;
    const int gr = ((slot & 15) - row - 8 * (cl & 1)) & 15;
    const int m = m0 + row;
    const int k = (cw0 + cl) * KCH + gr * 8;
    const uint32_t off = (uint32_t)(((int64_t)m * p.ldx + (int64_t)g * K + k) * 2);
    const bool ok = m < M && (FULL || cw0 + cl < c_end) && (!RG || k < K);
    if (m0 + (i * 64) / XS < M) lds_load16(rx, lds_addr(xw + i * 64), ok ? off : OOB);
  }
#pragma unroll
  for (int cl = WF; cl < CW; ++cl) wload(cl);

  // (4) pairs, each once its own loads (and everything issued before them) have landed
  pin_epilogue_args(p);                             // every load is issued
  const int half = r16 >> 3;                        // A rows / B columns 8..15: the pair's second chunk
  const int R = r16 & 7;                            // weight row of this lane (A operand)
  const int mx = r16 & 7;                           // X row of this lane (B operand)
  const int wsw = R >> 1;
  const uint8_t* eb = reinterpret_cast<const uint8_t*>(ew);
  int sh = 0;
  if constexpr (RG) sh = (int)((uint32_t)(erow * KB + cw0 * 4) & 3u);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto pair = [&](int pp) {
    const int cl = 2 * pp + half;
    const bool valid = FULL || cw0 + cl < c_end;
    const uint4* wt = ww + cl * WT + R * 8;
    const uint4 a = wt[q4 ^ wsw], b = wt[(4 + q4) ^ wsw];
    // the exponent bytes are read whatever the chunk (past the range they are zeros) and then
    // replaced by a unit factor: a lane-dependent condition around the LDS read would make the
    // compiler branch and wait on each read
    const int kb = (cw0 + cl) * 4 + (q4 >> 1);
    const int ei = (RG ? sh : 0) + cl * 4 + (q4 >> 1);
    const uint32_t b0 = eb[ei], b1 = eb[ei + 2];
    const float s0 = valid && (!RG || kb < KB) ? block_scale(b0) : 1.0f;
    const float s1 = valid && (!RG || kb + 2 < KB) ? block_scale(b1) : 1.0f;
    const uint4* xr = xw + mx * XS + cl * 16;
    const int rot = mx + 8 * (cl & 1);
    const bf16x8_t x0 = __builtin_bit_cast(bf16x8_t, xr[(2 * q4 + rot) & 15]);
    const bf16x8_t x1 = __builtin_bit_cast(bf16x8_t, xr[(2 * q4 + 1 + rot) & 15]);
    const bf16x8_t x2 = __builtin_bit_cast(bf16x8_t, xr[(8 + 2 * q4 + rot) & 15]);
    const bf16x8_t x3 = __builtin_bit_cast(bf16x8_t, xr[(9 + 2 * q4 + rot) & 15]);
    f32x4_t c = acc;
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.x, a.y, s0), x0, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(a.z, a.w, s0), x1, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.x, b.y, s1), x2, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(b.z, b.w, s1), x3, c, 0, 0, 0);
    acc = c;
  };
  wait_vmcnt_le<CW - 2>();
  pair(0);
  if constexpr (CP > 1) { wait_vmcnt_le<(CP > 1 ? CW - 4 : 0)>(); pair(1); }
  if constexpr (CP > 2) { wait_vmcnt_le<(CP > 2 ? CW - 6 : 0)>(); pair(2); }
  if constexpr (CP > 3) { wait_vmcnt_le<(CP > 3 ? CW - 8 : 0)>(); pair(3); }
  static_assert(CP <= 4, "pairs per wave");

  // (5) the two halves: lane l (q4 < 2, r16 < 8) holds D[4 q4 + v][r16] of the first chunks,
  //     lane l + 40 the matching D[8 + 4 q4 + v][8 + r16] of the second
  f32x4_t other;
#pragma unroll
  for (int v = 0; v < 4; ++v) other[v] = __shfl_down(acc[v], 40);
  acc += other;
  const bool useful = q4 < 2 && r16 < 8;
  const int slot = useful ? q4 * 8 + r16 : 0;

  // (6) waves along K: ascending-order sum through LDS. Wave 0 issues all its reads before the
  //     first add (a condition inside the loop would make each read a separate round trip).
  if constexpr (NWK > 1) {
    if (wk > 0 && useful) red[(wk - 1) * 16 + slot] = acc;
    __syncthreads();
    if (wk != 0) return;
    f32x4_t part[NWK - 1];
#pragma unroll
    for (int w = 1; w < NWK; ++w) part[w - 1] = red[(w - 1) * 16 + slot];
#pragma unroll
    for (int w = 1; w < NWK; ++w) acc += part[w - 1];
  }
  // (7) output: X row m0 + r16, weight rows n0 + 4 q4 .. + 3
  const int m = m0 + r16;
  const bool live = useful && m < M;
  const int n = n0 + 4 * q4;
  const size_t o = ((size_t)m * G + g) * N + n;
  if (FULL || (p.splits == 1 && !p.part)) {             // (FULL: one split; partials mode then
    if (live) {                                         // passes the workspace as an fp32 y)
      if (p.out_f32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + o) = acc;
      } else {
        const uint2 w2 = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) = w2;
      }
    }
    return;
  }
  float v[4];
  size_t off[4];
  int mr[4];
  bool lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = acc[i];
    off[i] = o + i;
    mr[i] = m;
    lv[i] = live;
  }
  combine_splits<4>(p, s, v, off, mr, lv);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lv[i]) store_out(p, off[i], v[i]);
}

// Split-K reduction for the tile kernel: Y = sum over s = 0, 1, ..., S-1 of the partials, added
// in that order in fp32, then rounded once to the output type. Four outputs per thread.
__global__ void __launch_bounds__(256)
reduce_splits_kernel(const float* __restrict__ part, void* __restrict__ y, int64_t n4, int splits,
                     int out_f32) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(part);
  f32x4_t a = p4[i];
  for (int s = 1; s < splits; ++s) a += p4[(int64_t)s * n4 + i];
  if (out_f32) {
    reinterpret_cast<f32x4_t*>(y)[i] = a;
  } else {
    reinterpret_cast<uint2*>(y)[i] = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
  }
}

// ---------------------------------------------------------------------------------------------
// configuration table
// ---------------------------------------------------------------------------------------------
typedef void (*KernelFn)(KParams);

enum Kind { STAGED = 0, DIRECT = 1, ROWS = 2, TILE = 3, DECODE = 4, SLAB = 5, PAIR = 6, PAIR_FULL = 7, ROWS_DMA = 8 };

struct Config {
  int MT, NT, NWM, NWN, NWK, CW;         // TILE: CW = chunks in flight; SLAB: CW = ring stages;
                                         // DECODE: MT = X rows
  KernelFn fn;
  int kind;                              // DIRECT, ROWS and DECODE kernels make one pass
  int row_scales = 0;                    // 1: exponents per weight row and 32 columns
  int TR = 16;                           // DECODE: real weight rows per 16-row MFMA tile (8 or 16)
  int ragged = 0;                        // DECODE: takes K that is not a multiple of 128
  int xg = 0;                            // XCDs per group of the XCD-grouped tile maps (G = 8 / xg)
};

#define CFG(MT, NT, NWN, NWK, CW) {MT, NT, 1, NWN, NWK, CW, gemm_kernel<MT, NT, NWN, NWK, CW>, STAGED}
#define DCFG(NT, NWN, NWK, CW) {1, NT, 1, NWN, NWK, CW, gemm_direct_kernel<NT, NWN, NWK, CW>, DIRECT}
#define RCFG(MT, NT, NWK, CW, D) {MT, NT, 1, 1, NWK, CW, gemm_rows_kernel<MT, NT, NWK, CW, D>, ROWS}
#define ECFG(NT, NWN, NWK, CW, XR) {XR, NT, 1, NWN, NWK, CW, gemm_decode_kernel<NT, NWN, NWK, CW, XR, 0, 16>, DECODE, 0, 16}
#define ERCFG(NT, NWN, NWK, CW, XR, TR) {XR, NT, 1, NWN, NWK, CW, gemm_decode_kernel<NT, NWN, NWK, CW, XR, 1, TR>, DECODE, 1, TR}
#define TCFG(MT, NT, NWM, NWN, D, GI) {MT, NT, NWM, NWN, 1, D, gemm_tile_kernel<MT, NT, NWM, NWN, D, GI>, TILE}
#define SCFG(MT, NT, NWM, NWN, NWK, S) {MT, NT, NWM, NWN, NWK, S, gemm_slab_kernel<MT, NT, NWM, NWN, NWK, S>, SLAB}
#define PCFG(NWK, CP, RG) {8, 1, 1, 1, NWK, 2 * CP, gemm_pair_kernel<NWK, CP, RG>, PAIR, 0, 8, RG}
#define PFCFG(NWK, CP) {8, 1, 1, 1, NWK, 2 * CP, gemm_pair_kernel<NWK, CP, false, true>, PAIR_FULL, 0, 8, 0}
#define PFWCFG(NWK, CP, WF) {8, 1, 1, 1, NWK, 2 * CP, gemm_pair_kernel<NWK, CP, false, true, WF>, PAIR_FULL, 0, 8, 0}
#define PFXCFG(NWK, CP, WF) {8, 1, 1, 1, NWK, 2 * CP, gemm_pair_kernel<NWK, CP, false, true, WF, true>, PAIR_FULL, 0, 8, 0, 4}
#define RDCFG(MT, NT, NWK, CW, D) {MT, NT, 1, 1, NWK, CW, gemm_rows_dma_kernel<MT, NT, NWK, CW, D>, ROWS_DMA}

const Config kConfigs[] = {
    CFG(1, 1, 4, 1, 4),   // 0  small: 64 rows, one wave per 16 rows, 4 chunks per wave
    CFG(1, 1, 1, 8, 4),   // 1  small: 16 rows, 8 waves along K
    CFG(1, 1, 1, 4, 4),   // 2  small: 16 rows, 4 waves along K
    CFG(1, 1, 2, 4, 2),   // 3  small: 32 rows
    CFG(1, 1, 1, 4, 2),   // 4  small: 16 rows, 4 waves x 2 chunks
    CFG(1, 1, 4, 1, 8),   // 5  small: 64 rows, 8 chunks per wave
    CFG(1, 1, 1, 2, 4),   // 6  small: 16 rows, 2 waves along K
    CFG(1, 1, 1, 1, 8),   // 7  small: 16 rows, one wave
    CFG(1, 1, 2, 2, 4),   // 8  small: 32 rows, 2x2 waves
    CFG(2, 1, 4, 1, 4),   // 9  mid: 32 x 64 tile
    CFG(4, 1, 4, 1, 2),   // 10 mid: 64 x 64 tile
    CFG(4, 2, 2, 1, 2),   // 11 mid: 64 x 64 tile, two n-subtiles per wave
    CFG(2, 2, 2, 2, 2),   // 12 mid: 32 x 64 tile, 2 waves along K
    CFG(1, 2, 2, 2, 2),   // 13 small: 16 x 64 tile, 2 n-subtiles per wave
    CFG(4, 2, 4, 1, 1),   // 14 mid: 64 x 128 tile
    CFG(2, 1, 2, 1, 4),   // 15 mid: 32 x 32 tile
    CFG(4, 1, 2, 1, 2),   // 16 mid: 64 x 32 tile
    CFG(1, 1, 2, 4, 4),   // 17 small: 32 rows, 4 waves along K, 4 chunks each
    CFG(1, 1, 4, 2, 4),   // 18 small: 64 rows, 2 waves along K
    DCFG(1, 1, 4, 4),     // 19 direct: 16 rows, 4 waves along K x 4 chunks
    DCFG(1, 1, 8, 4),     // 20 direct: 16 rows, 8 waves along K x 4 chunks
    DCFG(1, 1, 4, 2),     // 21 direct: 16 rows, 4 waves along K x 2 chunks
    DCFG(1, 2, 4, 2),     // 22 direct: 32 rows, 4 waves along K x 2 chunks
    DCFG(1, 1, 2, 4),     // 23 direct: 16 rows, 2 waves along K x 4 chunks
    DCFG(1, 1, 4, 8),     // 24 direct: 16 rows, 4 waves along K x 8 chunks
    DCFG(1, 2, 2, 4),     // 25 direct: 32 rows, 2 waves along K x 4 chunks
    DCFG(1, 4, 1, 4),     // 26 direct: 64 rows, 1 wave along K x 4 chunks
    DCFG(1, 1, 8, 2),     // 27 direct: 16 rows, 8 waves along K x 2 chunks
    DCFG(2, 1, 4, 4),     // 28 direct: 32 rows (2 subtiles per wave), 4 waves along K
    RCFG(1, 1, 8, 4, 4),  // 29 rows: 16 x 16 tile, 8 waves along K x 4 chunks, all in flight
    RCFG(1, 2, 8, 4, 4),  // 30 rows: 16 x 32 tile
    RCFG(2, 2, 8, 4, 2),  // 31 rows: 32 x 32 tile, two chunks in flight per wave
    RCFG(3, 2, 8, 4, 2),  // 32 rows: 48 x 32 tile
    RCFG(4, 2, 4, 8, 2),  // 33 rows: 64 x 32 tile, 4 waves along K x 8 chunks
    RCFG(2, 2, 8, 4, 4),  // 34 rows: 32 x 32 tile, all four chunks in flight
    RCFG(2, 1, 8, 4, 4),  // 35 rows: 32 x 16 tile
    RCFG(3, 2, 8, 4, 3),  // 36 rows: 48 x 32 tile, three chunks in flight
    RCFG(2, 2, 4, 8, 2),  // 37 rows: 32 x 32 tile, 4 waves along K x 8 chunks
    RCFG(3, 1, 8, 4, 4),  // 38 rows: 48 x 16 tile
    TCFG(1, 2, 1, 4, 7, 4),   // 39 tile: 16 x 128, 4 waves of 16 x 32, 7 stages, issued 4 at a time
    TCFG(1, 2, 2, 4, 6, 4),   // 40 tile: 32 x 128, 8 waves of 16 x 32, 6 stages
    TCFG(2, 2, 2, 4, 4, 2),   // 41 tile: 64 x 128, 8 waves of 32 x 32, 4 stages, 2 at a time
    TCFG(3, 2, 2, 4, 3, 1),   // 42 tile: 96 x 128, 8 waves of 48 x 32, 3 stages
    TCFG(4, 2, 2, 4, 3, 1),   // 43 tile: 128 x 128, 8 waves of 64 x 32, 3 stages
    TCFG(4, 4, 2, 2, 3, 1),   // 44 tile: 128 x 128, 4 waves of 64 x 64, 3 stages
    TCFG(2, 4, 2, 2, 4, 2),   // 45 tile: 64 x 128, 4 waves of 32 x 64, 4 stages
    TCFG(2, 2, 2, 2, 6, 4),   // 46 tile: 64 x 64, 4 waves of 32 x 32, 6 stages
    TCFG(3, 2, 2, 2, 4, 2),   // 47 tile: 96 x 64, 4 waves of 48 x 32, 4 stages
    TCFG(1, 4, 1, 2, 7, 4),   // 48 tile: 16 x 128, 2 waves of 16 x 64, 7 stages
    TCFG(1, 2, 1, 2, 8, 4),   // 49 tile: 16 x 64, 2 waves of 16 x 32, 8 stages
    TCFG(2, 2, 1, 4, 6, 4),   // 50 tile: 32 x 128, 4 waves of 32 x 32, 6 stages
    TCFG(1, 2, 1, 4, 7, 1),   // 51 tile: 16 x 128, 4 waves of 16 x 32, 7 stages, one at a time
    TCFG(1, 1, 1, 4, 12, 4),  // 52 tile: 16 x 64, 4 waves of 16 x 16, 12 stages
    TCFG(2, 2, 2, 4, 4, 1),   // 53 tile: 64 x 128, 8 waves of 32 x 32, 4 stages, one at a time
    ECFG(1, 1, 8, 4, 8),      // 54 decode: 8 rows of X x 16 weight rows, 8 waves along K x 4 chunks
    ECFG(1, 1, 4, 8, 8),      // 55 decode: 4 waves along K x 8 chunks
    ECFG(1, 2, 4, 4, 8),      // 56 decode: 32 weight rows, 4 waves along K x 4 chunks
    ECFG(1, 1, 4, 4, 8),      // 57 decode: 16 weight rows, 4 waves along K x 4 chunks
    ECFG(1, 2, 2, 4, 8),      // 58 decode: 32 weight rows, 2 waves along K x 4 chunks
    ECFG(1, 1, 4, 2, 8),      // 59 decode: 16 weight rows, 4 waves along K x 2 chunks
    ECFG(1, 1, 8, 2, 8),      // 60 decode: 16 weight rows, 8 waves along K x 2 chunks
    ECFG(1, 1, 4, 4, 16),     // 61 decode: 16 rows of X, 4 waves along K x 4 chunks
    RCFG(3, 2, 4, 8, 2),      // 62 rows: 48 x 32 tile, 4 waves along K x 8 chunks
    RCFG(2, 2, 4, 8, 4),      // 63 rows: 32 x 32 tile, 4 waves along K x 8 chunks, 4 in flight
    TCFG(1, 1, 1, 2, 16, 4),  // 64 tile: 16 x 32, 2 waves of 16 x 16, 16 stages
    TCFG(1, 1, 2, 2, 12, 4),  // 65 tile: 32 x 32, 4 waves of 16 x 16, 12 stages
    TCFG(3, 1, 1, 2, 9, 4),   // 66 tile: 48 x 32, 2 waves of 48 x 16, 9 stages
    TCFG(2, 1, 1, 2, 12, 4),  // 67 tile: 32 x 32, 2 waves of 32 x 16, 12 stages
    TCFG(2, 1, 2, 2, 7, 4),   // 68 tile: 64 x 32, 4 waves of 32 x 16, 7 stages
    SCFG(1, 1, 1, 2, 4, 4),   // 69 slab: 16 x 32, 8 waves (2 along N x 4 along K), 4 stages
    SCFG(1, 1, 2, 2, 2, 3),   // 70 slab: 32 x 32, 8 waves (2 x 2 x 2 along K), 3 stages
    SCFG(1, 2, 2, 1, 4, 3),   // 71 slab: 32 x 32, 8 waves (2 along M x 4 along K), 3 stages
    SCFG(3, 1, 1, 2, 4, 2),   // 72 slab: 48 x 32, 8 waves (2 along N x 4 along K), 2 stages
    SCFG(1, 1, 1, 4, 2, 3),   // 73 slab: 16 x 64, 8 waves (4 along N x 2 along K), 3 stages
    SCFG(1, 1, 2, 2, 1, 3),   // 74 slab: 32 x 32, 4 waves (2 x 2), 3 stages
    SCFG(1, 2, 1, 2, 4, 3),   // 75 slab: 16 x 64, 8 waves (2 along N x 4 along K), 3 stages
    // exponents per weight row and 32 columns (row-scale twins)
    ERCFG(1, 1, 8, 4, 8, 16),   // 76 decode: 8 rows of X x 16 weight rows, 8 waves along K x 4 chunks
    ERCFG(1, 1, 4, 2, 8, 16),   // 77 decode: 4 waves along K x 2 chunks
    ERCFG(1, 1, 4, 4, 16, 16),  // 78 decode: 16 rows of X, 4 waves along K x 4 chunks
    ERCFG(1, 1, 8, 2, 16, 16),  // 79 decode: 16 rows of X, 8 waves along K x 2 chunks
    ERCFG(1, 1, 8, 5, 8, 8),    // 80 decode: 8 weight rows, 8 waves along K x 5 chunks (40 in one pass)
    // the decode shapes of 54 and 59 for K that is not a multiple of 128
    {8, 1, 1, 1, 8, 4, gemm_decode_kernel<1, 1, 8, 4, 8, 0, 16, true>, DECODE, 0, 16, 1},   // 81
    {8, 1, 1, 1, 4, 2, gemm_decode_kernel<1, 1, 4, 2, 8, 0, 16, true>, DECODE, 0, 16, 1},   // 82
    // paired decode: 8 rows of X x 8 weight rows, each MFMA two chunks
    PCFG(8, 2, false),        // 83 pair: 8 waves along K x 4 chunks (32 chunks in one pass)
    PCFG(16, 1, false),       // 84 pair: 16 waves along K x 2 chunks
    PCFG(4, 4, false),        // 85 pair: 4 waves along K x 8 chunks
    PCFG(4, 2, false),        // 86 pair: 4 waves along K x 4 chunks
    PCFG(8, 1, false),        // 87 pair: 8 waves along K x 2 chunks
    PCFG(3, 1, false),        // 88 pair: 3 waves along K x 2 chunks (up to 6 chunks)
    PCFG(8, 2, true),         // 89 pair, K not a multiple of 128
    PCFG(3, 1, true),         // 90 pair, K not a multiple of 128, up to 6 chunks
    PCFG(4, 1, true),         // 91 pair, K not a multiple of 128, up to 8 chunks
    PCFG(4, 1, false),        // 92 pair: 4 waves along K x 2 chunks
    // paired decode over exactly the workgroup's chunks (K = 128 * NWK * CW, one split)
    PFCFG(8, 2),              // 93 pair, whole range: 8 waves x 4 chunks (K = 4096)
    PFCFG(4, 4),              // 94 pair, whole range: 4 waves x 8 chunks (K = 4096)
    PFCFG(3, 1),              // 95 pair, whole range: 3 waves x 2 chunks (K = 768)
    // register kernels with LDS-mode staging (bitwise the same sums as the ROWS entries alike)
    RDCFG(3, 2, 4, 8, 2),     // 96 rows, LDS-mode: 48 x 32 tile, 4 waves along K x 8 chunks, 2 in flight
    RDCFG(2, 2, 4, 8, 2),     // 97 rows, LDS-mode: 32 x 32 tile
    RDCFG(2, 2, 4, 8, 3),     // 98 rows, LDS-mode: 32 x 32 tile, 3 in flight
    RDCFG(3, 2, 8, 4, 1),     // 99 rows, LDS-mode: 48 x 32 tile, 8 waves along K x 4 chunks, 1 in flight
    RDCFG(2, 2, 8, 4, 1),     // 100 rows, LDS-mode: 32 x 32 tile, 8 waves along K
    RDCFG(1, 2, 8, 4, 2),     // 101 rows, LDS-mode: 16 x 32 tile, 8 waves along K, 2 in flight
    RDCFG(1, 2, 4, 8, 4),     // 102 rows, LDS-mode: 16 x 32 tile, 4 waves along K, 4 in flight
    TCFG(2, 2, 4, 4, 3, 1),   // 103 tile: 128 x 128, 16 waves of 32 x 32, 3 stages
    // decode workgroups for splits of few chunks (small LDS: several workgroups per CU)
    ECFG(1, 1, 4, 1, 8),      // 104 decode: 16 weight rows, 4 waves along K x 1 chunk
    ECFG(1, 1, 8, 1, 8),      // 105 decode: 16 weight rows, 8 waves along K x 1 chunk
    RDCFG(1, 1, 8, 4, 2),     // 106 rows, LDS-mode: 16 x 16 tile, 8 waves along K x 4 chunks
    RDCFG(1, 1, 4, 8, 2),     // 107 rows, LDS-mode: 16 x 16 tile, 4 waves along K x 8 chunks
    RDCFG(2, 1, 4, 8, 2),     // 108 rows, LDS-mode: 32 x 16 tile, 4 waves along K x 8 chunks
    PFWCFG(8, 2, 2),          // 109 pair, whole range (93) with the first pair's weights issued before X
    PFXCFG(8, 2, 0),          // 110 pair, whole range (93), one group per XCD half (G = 2 only)
    PFXCFG(8, 2, 2),          // 111 pair, whole range (109), one group per XCD half (G = 2 only)
    // the decode shape of 54 with a group per XCD half (G = 2) or quarter (G = 4)
    {8, 1, 1, 1, 8, 4, gemm_decode_kernel<1, 1, 8, 4, 8, 0, 16, false, 4>, DECODE, 0, 16, 0, 4},   // 112
    {8, 1, 1, 1, 8, 4, gemm_decode_kernel<1, 1, 8, 4, 8, 0, 16, false, 2>, DECODE, 0, 16, 0, 2},   // 113
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

int tree_levels(int splits) {
  int lv = 0;
  for (int c = splits; c > 1; c = (c + 1) >> 1) ++lv;
  return lv;
}

}  // namespace

int num_gemm_configs() { return kNumConfigs; }

int gemm_config_info(int cfg, int* out) {
  if (cfg < 0 || cfg >= kNumConfigs) return BSFP8_EINVAL;
  const Config& c = kConfigs[cfg];
  out[0] = c.kind == DECODE || c.kind == PAIR || c.kind == PAIR_FULL ? c.MT : 16 * c.MT * c.NWM;
  out[1] = c.TR * c.NT * c.NWN;
  out[2] = WAVE * c.NWM * c.NWN * c.NWK;
  out[3] = c.CW;
  out[4] = c.NWN;
  out[5] = c.NWK;
  out[6] = c.kind;
  out[7] = c.row_scales | (c.xg << 8);
  return BSFP8_OK;
}

int gemm_config_row_scales(int cfg) {
  return cfg >= 0 && cfg < kNumConfigs ? kConfigs[cfg].row_scales : 0;
}

int gemm_partials_order(const GemmPlan& p) {
  return kConfigs[p.cfg].kind == TILE ? BSFP8_SUM_ASCENDING : BSFP8_SUM_PAIRWISE;
}

int gemm_ws_needs_zero(const GemmPlan& p) { return p.splits > 1 && kConfigs[p.cfg].kind != TILE; }

size_t gemm_partials_bytes(const GemmShape& s, const GemmPlan& p) {
  return (size_t)p.splits * s.M * s.G * s.N * 4;
}

// Plan for an explicit configuration and chunks-per-split.
int plan_with(const GemmShape& s, int cfg, int cps, GemmPlan* plan) {
  if (cfg < 0 || cfg >= kNumConfigs) return BSFP8_EINVAL;
  const Config& c = kConfigs[cfg];
  GemmPlan p{};
  p.cfg = cfg;
  p.BM = c.kind == DECODE || c.kind == PAIR || c.kind == PAIR_FULL ? c.MT : 16 * c.MT * c.NWM;
  p.NB = c.TR * c.NT * c.NWN;
  if (s.N % p.NB) return BSFP8_ESHAPE;
  p.kchunks = (s.K + KCH - 1) / KCH;
  if (p.kchunks == 0) p.kchunks = 1;
  if (cps <= 0) return BSFP8_EINVAL;
  p.cps = cps < p.kchunks ? cps : p.kchunks;
  if (c.kind == PAIR_FULL && (p.kchunks != c.NWK * c.CW || p.cps != p.kchunks || s.K % KCH != 0))
    return BSFP8_EINVAL;                                        // exactly the workgroup's chunks
  if ((c.kind == DIRECT || c.kind == ROWS || c.kind == ROWS_DMA || c.kind == DECODE || c.kind == PAIR) &&
      p.cps > c.NWK * c.CW)
    return BSFP8_EINVAL;                                        // one pass
  if (c.kind == ROWS_DMA && s.K % KCH != 0) return BSFP8_EINVAL;  // whole chunks
  if ((c.kind == DECODE || c.kind == PAIR) && !c.ragged && s.K % KCH != 0) return BSFP8_EINVAL;  // whole words
  if (c.kind == TILE && (p.cps > TILE_MAX_CPS || s.K % KCH != 0)) return BSFP8_EINVAL;
  // slab kernel: K in whole chunks, splits begin on slab boundaries, one exponent word per lane
  if (c.kind == SLAB &&
      (s.K % KCH != 0 || p.cps > TILE_MAX_CPS || (p.cps < p.kchunks && p.cps % SLAB_CH != 0)))
    return BSFP8_EINVAL;
  p.splits = (p.kchunks + p.cps - 1) / p.cps;
  if (p.splits > 64) return BSFP8_EINVAL;
  p.mblocks = (s.M + p.BM - 1) / p.BM;
  p.nblocks = s.N / p.NB;
  if (c.xg && (s.G * c.xg != 8 || p.nblocks % c.xg != 0)) return BSFP8_EINVAL;   // its tile map needs both
  if (c.kind == TILE) {
    // fp32 partials [splits][M][G][N], summed by the reduce kernel
    if (p.splits > 1) p.ws_bytes = (size_t)p.splits * s.M * s.G * s.N * 4;
  } else if (p.splits > 1) {
    // one 64-bit slot per output element and tree node, the rows rounded up to whole 16s (the
    // slot layout groups each 16 x 16 output block)
    size_t nodes = 0;
    for (int c2 = p.splits; c2 > 1; c2 = (c2 + 1) >> 1) nodes += (size_t)(c2 >> 1);
    p.ws_bytes = nodes * (size_t)((s.M + 15) / 16 * 16) * s.G * s.N * 8;
  }
  *plan = p;
  return BSFP8_OK;
}

// Built-in choice (measured on MI355X, cold weights, graph replay). The plan depends on K only
// through ceil(K/128) and on whether K is a whole number of chunks; where that changes the kernel,
// the fp32 chain of every output stays the same, so K and K zero-padded inside the same chunk
// count give the same sums.
//  * Wide weights (at least 1024 tiles of 16 rows, e.g. an LM-head vocabulary shard): the tile
//    kernel, one split, for every row count (16 x 128 tiles up to 16 rows, 64 x 128 up to 64, then
//    128 x 128 on 16 waves, four per SIMD, 6-8% faster than 8 waves at 128 rows: the waves spend
//    a third of their cycles waiting for operands, and more of them overlap those waits). Each
//    output's fp32 sum is then the same ascending chain of chunks and MFMAs whatever the tile, so
//    a row's result does not depend on how many rows share the call.
//  * Decode rows (at most 8) over exactly 32 chunks on at most 256 eight-row tiles (wo_a at G = 2):
//    the paired decode kernel on the whole range, one workgroup per CU (up to 3 rows with the
//    first weight chunks issued before the X rows; with two groups from 3 rows on, each group on
//    its own half of the XCDs).
//  * Other decode rows (at most 8, or 16 with a long K): the decode kernel (everything streamed
//    into LDS, 8 rows of X per workgroup; with four groups, each on its own two XCDs); when K is
//    not whole 128-wide chunks its ragged
//    instances, which read zeros past K, so K zero-padded to whole chunks (576 -> 640) gives
//    bitwise the same Y.
//  * Few rows (at most 32): the one-pass register kernel with X rows in LDS, one 16-row block of X
//    per workgroup.
//  * More rows: the register kernel with 16-48 rows of X per workgroup, its chunks streamed
//    straight into LDS when K is whole chunks (no split while the K range fits one pass of 32
//    chunks).
int plan_gemm(const GemmShape& s, int path, int split_k, GemmPlan* plan, bool allow_pair) {
  const int kchunks = (s.K + KCH - 1) / KCH > 0 ? (s.K + KCH - 1) / KCH : 1;
  const bool n64 = (s.N % 64) == 0;
  const bool tile_ok = s.K % KCH == 0 && kchunks <= TILE_MAX_CPS && s.N % 128 == 0;
  const long long tiles16 = (long long)s.G * s.N / 16;
  int cfg, cps;
  if (tiles16 >= 1024) {
    cps = kchunks;
    if (tile_ok) cfg = s.M <= 16 ? 51 : s.M <= 64 ? 53 : 103;
    else if (path == PATH_SMALL || s.M <= 16) cfg = n64 ? 0 : 3;
    else if (s.M <= 32) cfg = n64 ? 9 : 15;
    else cfg = n64 ? 10 : 16;
  } else if (allow_pair && s.M <= 8 && s.K == 32 * KCH && split_k <= 1 && (long long)s.G * s.N / 8 <= 256) {
    // decode rows on at most 256 eight-row tiles over exactly 32 chunks: the paired kernel on the
    // whole range (one workgroup per CU, every MFMA computing two chunks). Up to 3 rows the first
    // pair's weight chunks go out before the X rows (3.77 against 3.87 us at 2 rows); from 4 rows
    // on the X rows go first (4.25 against 4.41 us at 6 rows). With two groups from 3 rows on,
    // each group's workgroups run on their own four XCDs (4.16 against 4.26 us at 6 rows, 4.06
    // against 4.16 at 4; at 2 rows 3.82 against 3.76, so not there). The sums are the same in
    // every variant.
    const bool xg = s.G == 2 && (s.N / 8) % 4 == 0;
    cfg = s.M <= 2 ? 109 : s.M <= 3 ? (xg ? 111 : 109) : (xg ? 110 : 93);
    cps = kchunks;
  } else if (s.M <= 8 || (s.M <= 16 && kchunks > 8)) {
    // decode kernel (8 rows of X per workgroup); for K that is not whole chunks its ragged
    // instance, whose last chunk reads zeros past K: K zero-padded to whole chunks gives bitwise
    // the same Y (as does the one-pass register kernel with the same waves and chunks, 21 / 20)
    const bool whole = s.K % KCH == 0;
    if (kchunks <= 8) {
      cfg = whole ? 59 : 82;         // 16 weight rows, 4 waves along K x 2 chunks
      cps = kchunks;
    } else {
      cfg = whole ? 54 : 81;         // 16 weight rows, 8 waves along K x 4 chunks
      cps = kchunks < 32 ? kchunks : 32;
      // four groups (wo_a at padded TP3): each group's workgroups on their own two XCDs, whose
      // L2s then fetch one group's activation rows instead of all four (5.15 against 5.60 us at
      // 2 rows, 5.29 against 5.53 at 6; no change with two groups at 16 rows)
      if (whole && s.G == 4 && (s.N / 16) % 2 == 0) cfg = 113;
    }
  } else if (path == PATH_SMALL || s.M <= 32) {
    if (s.M <= 16 && kchunks <= 8) {
      cfg = 25;                      // short K: 32 weight rows, 2 waves along K, no split
      cps = kchunks;
    } else if (s.M > 16 && s.K % KCH == 0 && kchunks <= 32) {
      cfg = 106;                     // 16 x 16 tiles staged through LDS, 8 waves along K x 4
      cps = kchunks;                 // chunks (bitwise the sums of the register kernel 20)
    } else {
      cfg = 20;                      // 16 weight rows, 8 waves along K x 4 chunks
      cps = 32;
    }
  } else {
    // K in whole chunks, at most 32 of them, up to 192 rows: the register kernel with LDS-mode
    // staging, 16 x 32 tiles with 8 waves along K x 4 chunks (M <= 64), 32 x 32 (<= 128) and
    // 48 x 32 (<= 192) with 4 waves along K x 8 chunks (the last two bitwise equal to the rows
    // kernel's 37 and 62). Up to 64 rows with a longer K: the slab kernel (16 x 32 tiles, X rows
    // read a kilobyte at a time), one split. Otherwise the rows kernel: 16 x 32 tiles, 8 waves
    // along K (M <= 64); 32 x 32 (<= 128), 48 x 32 (<= 192) and 64 x 32 tiles, 4 waves along K x 8
    // chunks.
    const bool whole = s.K % KCH == 0;
    if (whole && kchunks <= 32 && s.M <= 192) {
      cfg = s.M <= 64 ? 101 : s.M <= 128 ? 97 : 96;
      cps = kchunks;
    } else if (s.M <= 64 && whole && kchunks <= TILE_MAX_CPS) {
      cfg = 69;
      cps = kchunks;
    } else {
      cfg = s.M <= 64 ? 30 : s.M <= 128 ? 37 : s.M <= 192 ? 62 : 33;
      cps = kchunks < 32 ? kchunks : 32;
    }
  }
  if (split_k > 0) {
    cps = (kchunks + split_k - 1) / split_k;
    // An explicit split leaves each workgroup a few chunks: a workgroup sized for them (fewer
    // waves and chunk buffers, so several fit on a CU) instead of one sized for the whole range,
    // most of whose waves would sit idle while its LDS keeps the CU to one workgroup at a time.
    if (cfg == 54 || cfg == 59 || cfg == 113) cfg = cps <= 4 ? 104 : cps <= 8 ? 59 : cps <= 16 ? 60 : cfg;
    else if (cfg == 20 || cfg == 106) cfg = cps <= 8 ? 21 : cps <= 16 ? 19 : cfg;
  }
  const int st = plan_with(s, cfg, cps, plan);
  if (st != BSFP8_EINVAL) return st;
  // The one-pass choice cannot take this many chunks per split (an explicit split_k with a long
  // K): the staged kernel walks any K range in passes (16 rows of X, 4 waves along K).
  return plan_with(s, 2, cps, plan);
}

// The MXFP8-epilogue GEMM runs the plan bsfp8_gemm would pick for the same arguments, so its
// codes quantise exactly the fp32 outputs of that call.
int plan_gemm_mxfp8(const GemmShape& s, int split_k, GemmPlan* plan) {
  // not the paired kernel: its 8-row tiles hold a quarter of an MX block, while the 16-row
  // decode plan has a fused form that quantises whole blocks in the kernel
  return plan_gemm(s, s.M <= 8 ? PATH_SMALL : PATH_MID, split_k, plan, false);
}

// Built-in choice for weights with one exponent per row and 32 columns (a GEMV for up to 16
// rows, page "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row draft_main_proj): the
// decode kernel with row exponents and 8 rows of X per workgroup, with the waves and chunks the
// 32x32 plan uses for decode rows (so replicated block exponents give bitwise its results) up to
// 32 chunks; 33..40 chunks (K = 5120, the page's shape) run in one pass on half tiles; longer K
// is split over workgroups (the pairwise exchange combines the splits).
int plan_gemm_row32(const GemmShape& s, int split_k, GemmPlan* plan) {
  if (s.K % KCH != 0 || s.M > 16) return BSFP8_ESHAPE;
  const int kchunks = s.K / KCH;
  // 4 waves x 2 chunks, or 8 waves x 4 chunks; from 33 to 40 chunks, 8 waves x 5 chunks on
  // half tiles (8 weight rows per workgroup), which keeps the whole range in one pass
  const int cfg = kchunks <= 8 ? 77 : kchunks <= 32 ? 76 : kchunks <= 40 ? 80 : 76;
  const int cap = kchunks <= 8 ? 8 : kchunks <= 32 ? 32 : kchunks <= 40 ? 40 : 32;
  int cps = kchunks < cap ? kchunks : cap;
  if (split_k > 0) cps = (kchunks + split_k - 1) / split_k;
  return plan_with(s, cfg, cps, plan);
}

// Whether a configuration can quantise its own output to MXFP8 (one split): its workgroup tile
// has whole 32-column blocks that one wave can finish (the tile and rows kernels with an even
// number of 16-column tiles per wave, the slab kernel when every wave's partial tiles fit its
// ring). The kernels test the same conditions at compile time.
bool mx_fusable(const Config& c) {
  const int NB = c.TR * c.NT * c.NWN;
  if (NB % 32) return false;
  switch (c.kind) {
    case TILE:
    case ROWS:
    case ROWS_DMA:
      return c.NT % 2 == 0;
    case SLAB: {
      const int BM = 16 * c.MT * c.NWM, XG = BM * 64, WGR = NB * 32;
      return c.NWK * c.NWM * c.NWN * (c.MT * c.NT) * WAVE * 16 <= c.CW * (XG + WGR) * 16;
    }
    default:
      return false;
  }
}

int launch_gemm(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                const uint8_t* e, void* ws, void* y, int out_f32, hipStream_t stream, int partials,
                uint8_t* yq, uint8_t* ys) {
  if (yq && (p.splits != 1 || partials || !mx_fusable(kConfigs[p.cfg]))) return BSFP8_EINVAL;
  if (partials) {
    // fp32 results for a later kernel: the sum itself with one split, else every split's partial
    if (p.splits == 1) {
      y = ws;
      out_f32 = 1;
    }
  }
  KParams k{};
  k.x = x;
  k.q = q;
  k.e = e;
  k.y = y;
  k.slots = reinterpret_cast<unsigned long long*>(ws);
  k.ldx = s.ldx;
  const int64_t xb = ((int64_t)(s.M - 1) * s.ldx + (int64_t)s.G * s.K) * 2;
  const int64_t qb = (int64_t)s.G * s.N * s.K;
  // exponent bytes, rounded up to a whole word: the ragged decode instances read them as aligned
  // words, and with K / 32 not a multiple of 4 the last row's final word runs up to 3 bytes past
  // the array (inside the same page, as a page ends on a word; those bytes only reach blocks past
  // K, whose factors are replaced)
  const int64_t eb = ((kConfigs[p.cfg].row_scales ? (int64_t)s.G * s.N * (s.K / 32)
                                                  : (int64_t)s.G * (s.N / 32) * (s.K / 32)) + 3) & ~(int64_t)3;
  if (xb >= (int64_t)OOB || qb >= (int64_t)OOB || eb >= (int64_t)OOB) return BSFP8_ESHAPE;
  k.x_bytes = (uint32_t)xb;
  k.q_bytes = (uint32_t)qb;
  k.e_bytes = (uint32_t)eb;
  k.M = s.M;
  k.G = s.G;
  k.N = s.N;
  k.K = s.K;
  k.kchunks = p.kchunks;
  k.cps = p.cps;
  k.splits = p.splits;
  k.mblocks = p.mblocks;
  k.nblocks = p.nblocks;
  k.out_f32 = out_f32;
  if (partials && p.splits > 1 && kConfigs[p.cfg].kind != TILE) k.part = reinterpret_cast<float*>(ws);
  k.yq = yq;
  k.ys = ys;
  k.levels = tree_levels(p.splits);
  k.dm = make_fastdiv((uint32_t)p.mblocks);
  k.dn = make_fastdiv((uint32_t)p.nblocks);
  k.dg = make_fastdiv((uint32_t)s.G);
  const Config& c = kConfigs[p.cfg];
  const long long nwg = (long long)p.splits * s.G * p.nblocks * p.mblocks;
  if (nwg <= 0 || nwg > 0x7fffffffLL) return BSFP8_ESHAPE;
  k.nwg = (int)nwg;
  // the decode kernels take their tile from a three-dimensional grid (x = n-block, y = group,
  // z = split * mblocks + m-block); the others from the XCD-ordered index of a flat one
  const bool grid3 = c.kind == DECODE || c.kind == PAIR || c.kind == PAIR_FULL;
  const dim3 grid = grid3 ? dim3((unsigned)p.nblocks, (unsigned)s.G, (unsigned)(p.splits * p.mblocks))
                          : dim3((unsigned)nwg);
  hipLaunchKernelGGL(c.fn, grid, dim3(WAVE * c.NWM * c.NWN * c.NWK), 0, stream, k);
  if (c.kind == TILE && p.splits > 1 && !partials) {
    const int64_t n4 = (int64_t)s.M * s.G * s.N / 4;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(ws), y, n4, p.splits, out_f32);
  }
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
