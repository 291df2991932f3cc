// Device helpers shared by the bsfp8 HIP kernels (gemm.hip, mx.hip): kernel parameters, buffer
// loads (into VGPRs and, in LDS mode, straight into shared memory), the explicit wait on the
// vector memory counter, the LDS-ring barrier, the XCD-aware workgroup order and the pairwise
// split-K exchange. Not part of the public ABI.
#pragma once

#include "internal.h"

namespace bsfp8 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int KCH = 128;                 // K per chunk
constexpr int WAVE = 64;
constexpr uint32_t OOB = 0x80000000u;    // buffer offset beyond every descriptor's range
constexpr int RSRC_WORD3 = 0x00020000;   // raw buffer descriptor word 3 for gfx9-class GPUs

// Division by a divisor fixed at launch, without the integer-division sequence (a reciprocal on the
// vector unit and a chain of dependent scalar steps, some hundred cycles before a workgroup knows
// its tile): q = (n * mul) >> shift with mul = ceil(2^shift / d), shift = 31 + ceil(log2 d), set
// on the host (make_fastdiv). Exact for 0 <= n < 2^31: mul * d = 2^shift + e with 0 <= e < d, so
// n * mul / 2^shift = n / d + n * e / (d * 2^shift) and the second term is below 1 / d.
struct FastDiv {
  uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint32_t shift = 31 + l;
  return FastDiv{(uint32_t)(((1ull << shift) + d - 1) / d), shift};
}
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)(((uint64_t)(uint32_t)n * f.mul) >> f.shift);
}

struct KParams {
  const uint16_t* x;
  const uint8_t* q;
  const uint8_t* e;
  void* y;
  unsigned long long* slots;             // pairwise-combine slots (splits > 1)
  float* part;                           // non-null: each split stores its fp32 partial here,
                                         // [splits][M][G][N], for a later kernel to sum
  uint8_t* yq;                           // non-null (one split, 32-column tiles): MXFP8 output,
  uint8_t* ys;                           // codes [M][G*N] and scale bytes [M][G*N/32], not y
  int64_t ldx;
  uint32_t x_bytes, q_bytes, e_bytes;    // extents of the three buffer descriptors
  int M, G, N, K;
  int kchunks, cps, splits, mblocks, nblocks, out_f32;
  int nwg;                               // grid size (gridDim would be read from the dispatch packet)
  int levels;                            // tree levels of the pairwise combine (splits > 1)
  FastDiv dm, dn, dg;                    // division by mblocks, nblocks and G
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

__device__ __forceinline__ uint16_t to_bf16(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Weight stream: read once per call, so it is loaded non-temporally ("nt") and does not evict
// the activation slab, which every workgroup of the call re-reads from L2.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ uint4 load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL_NT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Logical workgroup index such that each XCD (hardware slot blockIdx % 8) owns a contiguous
// range of logical indices.
// (Branch-free: XCDs below `rem` hold per + 1 workgroups, the others per.)
__device__ __forceinline__ int xcd_logical(int i, int nwg) {
  const int xcd = i & 7, idx = i >> 3, per = nwg >> 3, rem = nwg & 7;
  return xcd * per + min(xcd, rem) + idx;
}

// Kernel arguments, in two steps. At entry, prefetch_args takes the fields the first loads' addresses
// need as inputs of empty asm statements: the compiler then issues their loads together (one round
// trip) instead of in dependent rounds, and waits for no other field. Once the kernel's loads are
// issued, pin_epilogue_args passes the fields the epilogue reads (output pointers, flags, sizes)
// through an empty asm as in-out operands: each is then the asm's output, not a load the compiler
// could repeat, so it stays in a register instead of being loaded again from the argument segment
// after the main loop (each such reload is a scalar memory round trip on the way to the stores).
__device__ __forceinline__ void prefetch_args(const KParams& p) {
  asm volatile("" ::"s"(p.x), "s"(p.q), "s"(p.e), "s"(p.ldx), "s"(p.x_bytes), "s"(p.q_bytes), "s"(p.e_bytes));
  asm volatile("" ::"s"(p.M), "s"(p.G), "s"(p.N), "s"(p.K), "s"(p.kchunks), "s"(p.cps), "s"(p.mblocks),
               "s"(p.nblocks), "s"(p.nwg));
}
__device__ __forceinline__ void pin_epilogue_args(KParams& p) {
  asm volatile("" : "+s"(p.y), "+s"(p.part), "+s"(p.yq), "+s"(p.ys), "+s"(p.slots));
  asm volatile("" : "+s"(p.splits), "+s"(p.out_f32), "+s"(p.M), "+s"(p.G), "+s"(p.N), "+s"(p.levels));
}
// (prefetch_args_only: the same loads at entry, for the staged multi-pass kernel, which keeps
// enough scalar state of its own that pinning the epilogue's fields makes it spill.)
__device__ __forceinline__ void prefetch_args_only(const KParams& p) {
  asm volatile("" ::"s"(p.x), "s"(p.q), "s"(p.e), "s"(p.y), "s"(p.slots), "s"(p.ldx));
  asm volatile("" ::"s"(p.x_bytes), "s"(p.q_bytes), "s"(p.e_bytes), "s"(p.M), "s"(p.G), "s"(p.N), "s"(p.K));
  asm volatile("" ::"s"(p.kchunks), "s"(p.cps), "s"(p.splits), "s"(p.mblocks), "s"(p.nblocks), "s"(p.out_f32),
               "s"(p.nwg));
}

// Workgroup -> (m-block, n-block, group, split) of the plan's tile order (m-blocks fastest), from
// the XCD-ordered logical index of a one-dimensional grid.
struct Tile {
  int mb, nb, g, s;
};
__device__ __forceinline__ Tile tile_of(const KParams& p) {
  int t = xcd_logical(blockIdx.x, p.nwg);
  Tile r;
  int q = fdiv(t, p.dm);
  r.mb = t - q * p.mblocks;
  t = q;
  q = fdiv(t, p.dn);
  r.nb = t - q * p.nblocks;
  t = q;
  q = fdiv(t, p.dg);
  r.g = t - q * p.G;
  r.s = q;
  return r;
}
// The same for a three-dimensional grid (x = n-block, y = group, z = split * mblocks + m-block),
// which the decode kernels use: the hardware hands each workgroup its indices, so nothing stands
// between the arguments and the first loads. A decode workgroup reads its own weight rows and its
// group's activations, which each XCD's L2 fetches on its first miss; with several groups the
// kernels' XCD-grouped instances remap (x, y) so that each XCD serves one group.
__device__ __forceinline__ Tile tile_of_grid(const KParams& p) {
  Tile r;
  r.nb = blockIdx.x;
  r.g = blockIdx.y;
  const int z = blockIdx.z;
  if (p.mblocks == 1) {
    r.mb = 0;
    r.s = z;
  } else {
    r.s = fdiv(z, p.dm);
    r.mb = z - r.s * p.mblocks;
  }
  return r;
}

// Exchange slot of output (m, c), c = g * N + n, inside one tree node's array of
// mp16 * 16 * G * N slots (mp16 = M rounded up to whole 16s, in 16s). The slots of one 16 x 16
// MFMA output block lie together, ordered (c / 16, m / 16, c % 4, c / 4 % 4, m % 16): the lanes
// of a wave exchanging one value of their accumulator (16 rows x four column groups) touch 64
// consecutive slots, four cache lines, where the element index would touch one line per row.
__device__ __forceinline__ size_t exch_slot(int m, int c, int mp16) {
  return ((((size_t)(c >> 4) * mp16 + (m >> 4)) * 4 + (c & 3)) << 6) + (((c >> 2) & 3) << 4) + (m & 15);
}

// Pairwise-combine tree over the split index for up to NV outputs of one lane (see the header
// comment). v[i] is this split's partial of output i, off[i] its element index (m * G * N + c) and
// mr[i] its row m, live[i] whether the lane owns it. All exchanges of one tree level are issued before any result
// is used, so a level costs one round trip to memory. On return live[i] says whether this lane
// finished output i (its total is then in v[i]). With p.part set the tree is left to a later
// kernel: split s stores its partials and finishes nothing.
template <int NV>
__device__ __forceinline__ void combine_splits(const KParams& p, int s, float (&v)[NV],
                                               const size_t (&off)[NV], const int (&mr)[NV], bool (&live)[NV]) {
  const size_t mgn = (size_t)p.M * p.G * p.N;
  if (p.part) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (live[i]) p.part[(size_t)s * mgn + off[i]] = v[i];
      live[i] = false;
    }
    return;
  }
  // node j of a level with cnt live partials combines splits 2j and 2j + 1; its slot array follows
  // those of the earlier levels (cnt / 2 nodes each)
  const int gn = p.G * p.N, mp16 = (p.M + 15) >> 4;
  const size_t node = (size_t)mp16 * 16 * gn;
  size_t slot[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) slot[i] = exch_slot(mr[i], (int)(off[i] - (size_t)mr[i] * gn), mp16);
  int idx = s, cnt = p.splits, level_base = 0;
  for (int lv = 0; lv < p.levels; ++lv) {
    if ((idx ^ 1) < cnt) {
      unsigned long long* base = p.slots + (size_t)(level_base + (idx >> 1)) * node;
      unsigned long long old[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        old[i] = live[i] ? atomicExch(base + slot[i], (1ull << 32) | __float_as_uint(v[i])) : 0ull;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (!live[i]) continue;
        if (old[i] == 0ull) {
          live[i] = false;                          // the partner finishes this node
        } else {
          v[i] = __uint_as_float((uint32_t)old[i]) + v[i];
          __hip_atomic_store(base + slot[i], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    level_base += cnt >> 1;
    idx >>= 1;
    cnt = (cnt + 1) >> 1;
  }
}

__device__ __forceinline__ void store_out(const KParams& p, size_t off, float v) {
  if (p.out_f32)
    reinterpret_cast<float*>(p.y)[off] = v;
  else
    reinterpret_cast<uint16_t*>(p.y)[off] = to_bf16(v);
}

constexpr int TILE_MAX_CPS = 64;                    // exponent staging: at most 64 chunks per split

// Workgroup barrier for the LDS ring: every LDS read of this wave has completed (lgkmcnt 0) and
// no memory access moves across it, but - unlike __syncthreads(), whose fence would also wait for
// the loads still streaming into the other stages - it does not wait for the vector memory
// counter.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer loads in LDS mode: lane l's bytes land at LDS address lds + l*size (lds is wave-uniform
// and travels in M0; the compiler cannot prove that values derived from the wave index are
// uniform, hence the readfirstlane). Written as inline assembly so that the compiler neither
// reorders them nor adds waits of its own for them; the kernel counts them itself with
// wait_vmcnt_le. (With __builtin_amdgcn_raw_ptr_buffer_load_lds the compiler cannot tell which
// ring stage or chunk buffer a load fills, so it waits for every LDS-mode load in flight before
// the first LDS read that might alias one: an s_waitcnt vmcnt(0) inside each ring loop, and
// before every chunk but the first of the decode kernel, which would serialise the streams.)
// M0 is a register the compiler reserves, so each load saves it into a scratch SGPR, sets it,
// issues the load and puts the saved value back: nothing the compiler may keep in M0 changes
// across the statement, and M0 is not on any clobber list. The s_nop gives the one wait state an
// LDS-mode load needs after an SALU write of M0.
typedef uint32_t lds_addr_t;
template <typename T>
__device__ __forceinline__ lds_addr_t lds_addr(const T* p) {
  return (lds_addr_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, lds_addr_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void lds_load16_stream(__amdgpu_buffer_rsrc_t r, lds_addr_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, lds_addr_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(r) : "memory");
}

// Wait until at most N of this wave's vector memory loads are outstanding (loads complete in
// order); no memory access of the kernel moves across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// e4m3 codes by the hardware's conversions, two values per instruction, round half to even:
//  * e4m3x4: four fp32 values with |v| <= 448 (v_cvt_pk_fp8_f32), byte i = value i;
//  * e4m3x2_bf16: a bf16 pair divided by 2^k, k = the scale operand's exponent field - 127 (field
//    0 reads as 2^-127; v_cvt_scalef32_pk_fp8_bf16), for results within +-448, in bits 0..15.
// Both were compared on the GPU with an integer RNE encoder written from the e4m3 definition
// (ties to the even code, subnormal quantum 2^-9, magnitudes below 2^-10 to a signed zero): the
// first over every fp32 value in [-448, 448], the second over every finite bf16 value and every
// k in [-127, 127]; no difference.
typedef short s16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t pair, float scale) {
  const s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2_t{0, 0}, __builtin_bit_cast(bf16x2_t, pair),
                                                             scale, false);
  return (uint32_t)(uint16_t)r[0];
}

// One MX block (32 consecutive outputs of a row, OCP MX v1.0 MXFP8 rule) held by the four lanes
// r16 + 16*q4 of a wave, eight fp32 values each: lo = columns 4*q4 .. +3, hi = 16 + 4*q4 .. +3 of
// the block. Returns the lane's eight e4m3 codes (lo in the first dword) and the block's scale
// byte: s = floor(log2 amax) - 8 from the fp32 exponent field, clamped below at -127; values
// scaled by the exact power of two, saturated at +-448 and rounded to nearest even (e4m3x4); a
// block holding inf or NaN gets byte 255 and NaN codes. Every lane of the wave must take part.
__device__ __forceinline__ uint8_t mx_block_codes(const f32x4_t& lo, const f32x4_t& hi, uint32_t& c_lo,
                                                  uint32_t& c_hi) {
  uint32_t u[8], amax = 0, nonfinite = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u[i] = __float_as_uint(i < 4 ? lo[i] : hi[i - 4]);
    const uint32_t mag = u[i] & 0x7FFFFFFFu;
    nonfinite |= mag >= 0x7F800000u ? 1u : 0u;
    amax = mag > amax ? mag : amax;
  }
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)amax, off);
    amax = o > amax ? o : amax;
    nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off);
  }
  const int E = (int)(amax >> 23);
  int s = E == 0 ? -127 : E - 135;
  s = s < -127 ? -127 : s;
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = fminf(fmaxf(ldexpf(__uint_as_float(u[i]), -s), -448.f), 448.f);
  c_lo = e4m3x4(sv[0], sv[1], sv[2], sv[3]);
  c_hi = e4m3x4(sv[4], sv[5], sv[6], sv[7]);
  if (nonfinite) {                                  // NaN codes carrying each entry's sign
    uint32_t nl = 0, nh = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nl |= ((u[i] >> 31) ? 0xFFu : 0x7Fu) << (8 * i);
      nh |= ((u[i + 4] >> 31) ? 0xFFu : 0x7Fu) << (8 * i);
    }
    c_lo = nl;
    c_hi = nh;
  }
  return nonfinite ? (uint8_t)255 : (uint8_t)(s + 127);
}

// Store one lane's share of an MX block of row m, group g, starting at output column n0 (a
// multiple of 32): codes [M][G*N], scale bytes [M][G*N/32].
__device__ __forceinline__ void store_mx_block(uint8_t* yq, uint8_t* ys, int m, int g, int G, int N, int n0,
                                               int q4, uint32_t c_lo, uint32_t c_hi, uint8_t scale) {
  uint8_t* row = yq + ((size_t)m * G + g) * N + n0;
  *reinterpret_cast<uint32_t*>(row + q4 * 4) = c_lo;
  *reinterpret_cast<uint32_t*>(row + 16 + q4 * 4) = c_hi;
  if (q4 == 0) ys[((size_t)m * G + g) * (N / 32) + n0 / 32] = scale;
}

}  // namespace
}  // namespace bsfp8
