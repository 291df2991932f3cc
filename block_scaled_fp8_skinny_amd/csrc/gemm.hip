// Small-M block-scaled fp8 weight GEMM for gfx950 (MI355X).
//
// Computes Y[m][g][n] = sum_k X[m][g*K + k] * W[g][n][k], where the weight is stored as e4m3
// codes plus one exponent byte per 32x32 block and each tile is rebuilt exactly in bf16
// registers before a bf16 MFMA with fp32 accumulation (page
// "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py": kernels _wo_a_partial_w8 and
// _wo_a_mid_kernel; the split-K partials are summed in a fixed order, as its mid-path notes ask).
//
// Design (gfx950, wave64):
//  * MFMA v_mfma_f32_16x16x32_bf16 with the WEIGHT as the A operand (16 rows of W) and X^T as
//    the B operand (16 rows of X), so D[n][m] holds four consecutive n per lane: one 8- or
//    16-byte store per lane in the epilogue.
//  * K is walked in 128-wide chunks. In a chunk each lane loads two 16-byte pieces of one weight
//    row (k offsets 16*q and 64 + 16*q for lane group q = lane/16), i.e. a wave reads whole
//    128-byte lines of 16 rows, straight from HBM into VGPRs.
//  * Dequant is v_cvt_scalef32_pk_bf16_fp8: 2 codes -> 2 bf16 scaled by the block factor in one
//    instruction, exact for every code and exponent byte 0..254 (checked on the hardware).
//  * X and the exponent bytes of the workgroup's K range are staged in LDS; X is stored in MFMA
//    fragment order (1 KB per 64-lane fragment), so every fragment read is one conflict-free
//    ds_read_b128 per lane.
//  * Waves of a workgroup split the n rows (NWN) and the chunks (NWK); partial tiles of the NWK
//    waves are summed through LDS in ascending wave order. Workgroups can further split K
//    (splits > 1): each writes fp32 partials, and the last to arrive at a tile (an atomic arrival
//    counter) sums them in ascending split order and stores Y. The order never depends on which
//    workgroup arrives last, so results are bitwise reproducible.
//  * The map chunk -> (split, wave, step) depends only on the chunk index and the plan, not on
//    K, so zero-padding K inside the same number of chunks leaves every fp32 sum unchanged.
//  * Workgroup ids are remapped so that consecutive logical tiles run on the same XCD
//    (workgroups are dealt round-robin over the 8 XCDs): splits sharing an X slab and m-blocks
//    sharing a weight tile hit the same L2.

#include "internal.h"

namespace bsfp8 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int KCH = 128;   // K per chunk
constexpr int WAVE = 64;

struct KParams {
  const uint16_t* x;
  int64_t ldx;
  const uint8_t* q;
  const uint8_t* e;
  void* y;
  float* part;
  uint32_t* counters;
  int M, G, N, K;
  int kchunks, cps, splits, mblocks, nblocks, out_f32;
};

__device__ __forceinline__ uint32_t bits_of(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Eight e4m3 codes (two dwords, k order = byte order) times the block factor -> eight bf16.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t lo, uint32_t hi, float scale) {
  u32x4_t r;
  r[0] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false));
  r[1] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true));
  r[2] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false));
  r[3] = bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true));
  return __builtin_bit_cast(bf16x8_t, r);
}

// Block factor 2^(b-127) as the fp32 whose exponent field is b (the convert reads the exponent).
__device__ __forceinline__ float block_scale(uint32_t b) { return __uint_as_float(b << 23); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round half to even
  return bits_of(v);
}

// Logical workgroup index such that each XCD (hardware slot blockIdx % 8) owns a contiguous
// range of logical indices.
__device__ __forceinline__ int xcd_logical(int i, int nwg) {
  const int xcd = i & 7, idx = i >> 3, per = nwg >> 3, rem = nwg & 7;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

template <int MT, int NT, int NWN, int NWK, int CW>
__global__ void __launch_bounds__(WAVE * NWN * NWK)
gemm_kernel(KParams p) {
  constexpr int NTHR = WAVE * NWN * NWK;
  constexpr int BM = 16 * MT;
  constexpr int NB = 16 * NT * NWN;
  constexpr int PCH = NWK * CW;                     // chunks per pass
  constexpr int XBYTES = PCH * 4 * MT * 1024;       // X fragments of one pass
  constexpr int EROWS = NB >= 32 ? NB / 32 : 1;
  constexpr int ECOLS = PCH * 4;
  constexpr int XUNITS = BM * PCH * 16;             // 16-byte pieces of the pass's X tile
  static_assert(XUNITS % NTHR == 0, "X staging must divide evenly over the threads");
  constexpr int XPT = XUNITS / NTHR;
  constexpr int REDBYTES = (NWK - 1) * NWN * MT * NT * WAVE * 16;
  static_assert(REDBYTES <= XBYTES, "the reduction buffer aliases the X buffer");

  __shared__ __attribute__((aligned(16))) uint8_t x_lds[XBYTES];
  __shared__ uint8_t e_lds[EROWS * ECOLS];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wk = wave / NWN;
  const int q4 = lane >> 4, r16 = lane & 15;

  int t = xcd_logical(blockIdx.x, gridDim.x);
  const int mb = t % p.mblocks;
  t /= p.mblocks;
  const int nb = t % p.nblocks;
  t /= p.nblocks;
  const int g = t % p.G;
  const int s = t / p.G;

  const int n0 = nb * NB, m0 = mb * BM;
  const int c_begin = s * p.cps;
  const int c_end = min(c_begin + p.cps, p.kchunks);
  const int npass = (c_end - c_begin + PCH - 1) / PCH;
  const int K = p.K, M = p.M;

  const uint8_t* qg = p.q + (size_t)g * p.N * K;
  const uint8_t* eg = p.e + (size_t)g * (p.N / 32) * (K / 32);
  const uint16_t* xg = p.x + (size_t)g * K;
  const int nrow = n0 + wn * 16 * NT + r16;         // + 16*ts: the weight row this lane loads
  const int erow0 = n0 / 32;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int pass = 0; pass < npass; ++pass) {
    const int pc0 = c_begin + pass * PCH;
    const int pch = min(PCH, c_end - pc0);
    if (pass) __syncthreads();                      // LDS of the previous pass fully consumed

    // (1) X pieces of this pass (L2-resident, issued first so the waits below cover them only)
    uint4 xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int u = tid + i * NTHR;
      const int ml = u / (PCH * 16), kl = (u % (PCH * 16)) * 8;
      const int m = m0 + ml, k = pc0 * KCH + kl;
      xv[i] = make_uint4(0, 0, 0, 0);
      if (m < M && kl < pch * KCH && k < K)
        xv[i] = *reinterpret_cast<const uint4*>(xg + (size_t)m * p.ldx + k);
    }
    // (2) exponent bytes of this pass
    uint32_t ev = 0;
    static_assert(EROWS * ECOLS <= NTHR, "one exponent byte per thread");
    const bool e_thread = tid < EROWS * ECOLS;
    if (e_thread) {
      const int er = tid / ECOLS, ec = tid % ECOLS;
      const int kb = pc0 * 4 + ec;
      if (ec < pch * 4 && kb < K / 32) ev = eg[(size_t)(erow0 + er) * (K / 32) + kb];
    }
    // (3) this wave's weight pieces, streamed from HBM into registers
    uint4 wv[CW][NT][2];
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int cp = wk + j * NWK;
#pragma unroll
      for (int ts = 0; ts < NT; ++ts)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = (pc0 + cp) * KCH + h * 64 + q4 * 16;
          wv[j][ts][h] = make_uint4(0, 0, 0, 0);
          if (cp < pch && k < K)
            wv[j][ts][h] = *reinterpret_cast<const uint4*>(qg + (size_t)(nrow + ts * 16) * K + k);
        }
    }
    // (4) stage X in fragment order and the exponents
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int u = tid + i * NTHR;
      const int ml = u / (PCH * 16), kl = (u % (PCH * 16)) * 8;
      const int cp = kl / KCH, kk = kl % KCH;
      const int jj = (kk / 64) * 2 + ((kk % 16) / 8);
      const int fl = ((kk % 64) / 16) * 16 + (ml % 16);
      *reinterpret_cast<uint4*>(x_lds + ((((cp * 4 + jj) * MT + ml / 16) * 64 + fl) * 16)) = xv[i];
    }
    if (e_thread) e_lds[tid] = (uint8_t)ev;
    __syncthreads();

    // (5) dequant + MFMA, chunk by chunk in a fixed order
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int cp = wk + j * NWK;
      if (cp < pch) {
#pragma unroll
        for (int ts = 0; ts < NT; ++ts) {
          const int er = (nrow + ts * 16) / 32 - erow0;
          const float sc0 = block_scale(e_lds[er * ECOLS + cp * 4 + (q4 >> 1)]);
          const float sc1 = block_scale(e_lds[er * ECOLS + cp * 4 + 2 + (q4 >> 1)]);
          const uint4 a = wv[j][ts][0], b = wv[j][ts][1];
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
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < NWK; ++w)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ts = 0; ts < NT; ++ts)
            acc[mt][ts] += red[((((w - 1) * NWN + wn) * MT + mt) * NT + ts) * WAVE + lane];
    }
  }

  const int G = p.G, N = p.N;
  if (p.splits == 1) {
    if (wk == 0) {
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
              uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + off) = o;
            }
          }
        }
      }
    }
    return;
  }

  // splits > 1: publish this split's partial tile, then the last arriver reduces.
  if (wk == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + mt * 16 + r16;
      if (m < M) {
#pragma unroll
        for (int ts = 0; ts < NT; ++ts) {
          const int n = n0 + wn * 16 * NT + ts * 16 + q4 * 4;
          *reinterpret_cast<f32x4_t*>(p.part + (((size_t)s * M + m) * G + g) * N + n) = acc[mt][ts];
        }
      }
    }
  }
  __threadfence();                                  // release: partials visible device-wide
  __syncthreads();
  const int tile = (g * p.nblocks + nb) * p.mblocks + mb;
  if (tid == 0) {
    const uint32_t prev = atomicAdd(p.counters + tile, 1u);
    s_last = (prev == (uint32_t)(p.splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();                                  // acquire: see every split's partial
  const int rows = min(BM, M - m0);
  constexpr int C4 = NB / 4;
  for (int idx = tid; idx < rows * C4; idx += NTHR) {
    const int m = m0 + idx / C4, n = n0 + (idx % C4) * 4;
    const size_t stride = (size_t)M * G * N;
    const float* src = p.part + ((size_t)m * G + g) * N + n;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
    for (int sp = 1; sp < p.splits; ++sp) v += *reinterpret_cast<const f32x4_t*>(src + sp * stride);
    const size_t off = ((size_t)m * G + g) * N + n;
    if (p.out_f32) {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(p.y) + off) = v;
    } else {
      uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + off) = o;
    }
  }
  if (tid == 0) p.counters[tile] = 0;               // ready for the next call
}

// ---------------------------------------------------------------------------------------------
// configuration table
// ---------------------------------------------------------------------------------------------
typedef void (*KernelFn)(KParams);

struct Config {
  int MT, NT, NWN, NWK, CW;
  KernelFn fn;
};

#define CFG(MT, NT, NWN, NWK, CW) {MT, NT, NWN, NWK, CW, gemm_kernel<MT, NT, NWN, NWK, CW>}

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
    CFG(4, 1, 4, 1, 4),   // 10 mid: 64 x 64 tile
    CFG(4, 2, 2, 1, 2),   // 11 mid: 64 x 64 tile, two n-subtiles per wave
    CFG(2, 2, 2, 2, 2),   // 12 mid: 32 x 64 tile, 2 waves along K
    CFG(1, 2, 2, 2, 2),   // 13 small: 16 x 64 tile, 2 n-subtiles per wave
    CFG(4, 2, 4, 1, 2),   // 14 mid: 64 x 128 tile
    CFG(2, 1, 2, 1, 4),   // 15 mid: 32 x 32 tile
    CFG(4, 1, 2, 1, 4),   // 16 mid: 64 x 32 tile
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace

int num_gemm_configs() { return kNumConfigs; }

int gemm_config_info(int cfg, int* out) {
  if (cfg < 0 || cfg >= kNumConfigs) return BSFP8_EINVAL;
  const Config& c = kConfigs[cfg];
  out[0] = 16 * c.MT;
  out[1] = 16 * c.NT * c.NWN;
  out[2] = WAVE * c.NWN * c.NWK;
  out[3] = c.CW;
  return BSFP8_OK;
}

// Plan for an explicit configuration and chunks-per-split.
int plan_with(const GemmShape& s, int cfg, int cps, GemmPlan* plan) {
  if (cfg < 0 || cfg >= kNumConfigs) return BSFP8_EINVAL;
  const Config& c = kConfigs[cfg];
  GemmPlan p{};
  p.cfg = cfg;
  p.BM = 16 * c.MT;
  p.NB = 16 * c.NT * c.NWN;
  if (s.N % p.NB) return BSFP8_ESHAPE;
  p.kchunks = (s.K + KCH - 1) / KCH;
  if (p.kchunks == 0) p.kchunks = 1;
  if (cps <= 0) return BSFP8_EINVAL;
  p.cps = cps < p.kchunks ? cps : p.kchunks;
  p.splits = (p.kchunks + p.cps - 1) / p.cps;
  p.mblocks = (s.M + p.BM - 1) / p.BM;
  p.nblocks = s.N / p.NB;
  if (p.splits > 1) {
    const size_t tiles = (size_t)s.G * p.nblocks * p.mblocks;
    p.counter_bytes = (tiles * 4 + 255) & ~(size_t)255;
    p.ws_bytes = p.counter_bytes + (size_t)p.splits * s.M * s.G * s.N * 4;
  }
  *plan = p;
  return BSFP8_OK;
}

// Built-in choice. The key uses ceil(K/128), never K itself, so K and K zero-padded inside the
// same chunk count get the same plan (and the same fp32 sums).
int plan_gemm(const GemmShape& s, int path, int split_k, GemmPlan* plan) {
  const int kchunks = (s.K + KCH - 1) / KCH > 0 ? (s.K + KCH - 1) / KCH : 1;
  const bool n64 = (s.N % 64) == 0;
  int cfg, cps;
  if (path == PATH_SMALL || s.M <= 16) {
    if (kchunks <= 8) {
      cfg = 7;                       // short K: one wave per 16 rows, no split
      cps = kchunks;
    } else {
      cfg = n64 ? 0 : 3;
      cps = 4;
    }
  } else if (s.M <= 32) {
    cfg = n64 ? 9 : 15;
    cps = 4;
  } else {
    cfg = n64 ? 10 : 16;
    cps = 4;
  }
  if (split_k > 0) cps = (kchunks + split_k - 1) / split_k;
  return plan_with(s, cfg, cps, plan);
}

int launch_gemm(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                const uint8_t* e, void* ws, void* y, int out_f32, hipStream_t stream) {
  KParams k;
  k.x = x;
  k.ldx = s.ldx;
  k.q = q;
  k.e = e;
  k.y = y;
  k.counters = reinterpret_cast<uint32_t*>(ws);
  k.part = p.splits > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + p.counter_bytes) : nullptr;
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
  const Config& c = kConfigs[p.cfg];
  const long long nwg = (long long)p.splits * s.G * p.nblocks * p.mblocks;
  if (nwg <= 0 || nwg > 0x7fffffffLL) return BSFP8_ESHAPE;
  hipLaunchKernelGGL(c.fn, dim3((unsigned)nwg), dim3(WAVE * c.NWN * c.NWK), 0, stream, k);
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
