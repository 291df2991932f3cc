// Measurement aid: the plain-read floor of a weight stream on gfx950.
//
// The GEMM's cost at decode row counts is the time to stream its weight bytes from HBM plus a
// fixed launch and first-byte latency. This kernel does only the first part of that work: it
// reads `bytes` of a buffer once, with the GEMM's load shape (16 bytes per lane, one contiguous
// kilobyte per wave load, non-temporal, every load of a workgroup's share in flight at once, up to
// twelve per wave), and folds what it read into one word per lane, which it stores only if it
// matches a constant no realistic data hits (the store keeps every lane's loads alive; the sink is
// written at most once per workgroup in practice).
// Timed on the same distinct weight copies as the GEMM, it is the floor a GEMM of that size can
// approach on this machine; with bytes = 0 it is the cost of a launch. With an output buffer it
// also writes `out_bytes` there (16 bytes per lane, each workgroup one contiguous share, after
// its reads): the read + write floor of a GEMM that streams those bytes and stores that many
// output bytes (a kernel that stores pays for its writes and their completion at its end). With a
// slab, every workgroup also reads its group's slab whole (one kilobyte per wave load, straight
// into LDS, as the GEMMs read the activation rows of their group), all of it before its share
// or, in read_floor_il_kernel, spread over the steps of its share: the floor of a GEMM whose
// workgroups each also read those shared, cache-resident bytes.
#include "device.h"

namespace bsfp8 {
namespace {

constexpr int FLOOR_WAVES = 8;
constexpr int FLOOR_MAX_L = 12;                     // loads per wave per step, at most
constexpr uint32_t FLOOR_MAGIC = 0x9E3779B9u;

// L loads per wave per step: a workgroup's share is walked in steps of L * 8 KB, each wave's load u
// of a step at kilobyte u * 8 + wave, every load of a step issued before any is used. The launch
// picks the smallest L that covers a share in one step (every decode size), else L = 12 and several
// steps. Loads past the share (the last step's tail) read at the out-of-range offset.
template <int L>
__global__ void __launch_bounds__(WAVE * FLOOR_WAVES)
read_floor_kernel(const uint8_t* p, uint32_t bytes, uint32_t per_wg, uint32_t steps, const uint8_t* slab,
                  uint32_t slab_bytes, uint32_t slab_groups, uint32_t* sink, uint4* out, uint32_t out16,
                  uint32_t out_per_wg16) {
  // every argument the loads need, fetched in one batch (left to itself the compiler fetched the
  // buffer pointer only after a bounds test: a second dependent round trip), and the ones the end
  // needs held in registers rather than fetched after the reads
  asm volatile("" ::"s"(p), "s"(bytes), "s"(per_wg), "s"(steps), "s"(slab), "s"(slab_bytes), "s"(slab_groups));
  asm volatile("" : "+s"(sink), "+s"(out), "+s"(out16), "+s"(out_per_wg16));
  __shared__ uint4 slab_lds[FLOOR_WAVES * WAVE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (slab_bytes) {
    // the group's slab, wave w taking kilobytes w, w + 8, ... (every load lands in this wave's
    // kilobyte of LDS; the contents are never read)
    const uint32_t grp = (uint32_t)(((uint64_t)blockIdx.x * slab_groups) / gridDim.x);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)slab, 0, (int)(slab_bytes * slab_groups), RSRC_WORD3);
    const lds_addr_t dst = lds_addr(slab_lds + wave * WAVE);
    for (uint32_t o = (uint32_t)wave * 1024u; o < slab_bytes; o += FLOOR_WAVES * 1024u) {
      const uint32_t off = o + (uint32_t)lane * 16u;
      lds_load16(rs, dst, off < slab_bytes ? grp * slab_bytes + off : OOB);
    }
  }
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)bytes, RSRC_WORD3);
  const uint32_t begin = blockIdx.x * per_wg;
  const uint32_t end = min(begin + per_wg, bytes);
  const uint32_t first = begin + (uint32_t)wave * 1024u + (uint32_t)lane * 16u;
  uint32_t acc = 0;
  for (uint32_t st = 0; st < steps; ++st) {
    uint4 v[L];
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const uint32_t off = first + (st * L + (uint32_t)u) * FLOOR_WAVES * 1024u;
      v[u] = load16_stream(r, off < end ? off : OOB);
    }
    __builtin_amdgcn_sched_barrier(0);             // every load of the step in flight before any is used
#pragma unroll
    for (int u = 0; u < L; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the slab loads write LDS: none may still be in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (out) {
    const uint32_t b = blockIdx.x * out_per_wg16, e = min(b + out_per_wg16, out16);
    // long shares are streamed with non-temporal stores, as the dequantiser writes its output (a
    // 33.5 MB write took 8.8 against 9.7 us with them); short ones with plain stores, as the GEMMs
    // write theirs (non-temporal stores of 24 KB took 0.3 us longer to complete)
    if (out_per_wg16 >= 1024) {
      const u32x4_t a4 = {acc, acc, acc, acc};
      for (uint32_t i = b + threadIdx.x; i < e; i += WAVE * FLOOR_WAVES)
        __builtin_nontemporal_store(a4, reinterpret_cast<u32x4_t*>(out + i));
    } else {
      for (uint32_t i = b + threadIdx.x; i < e; i += WAVE * FLOOR_WAVES) out[i] = make_uint4(acc, acc, acc, acc);
    }
  } else if (acc == FLOOR_MAGIC) {
    sink[blockIdx.x] = acc;
  }
}

// The same with the slab spread over the steps of a share of several steps: wave w's slab loads
// (load i at kilobyte w + 8i) go out slab_per_step at a time, each group just before the share
// loads of its step, as a GEMM issues each chunk's activation rows before its weights.
template <int L>
__global__ void __launch_bounds__(WAVE * FLOOR_WAVES)
read_floor_il_kernel(const uint8_t* p, uint32_t bytes, uint32_t per_wg, uint32_t steps, const uint8_t* slab,
                     uint32_t slab_bytes, uint32_t slab_groups, uint32_t slab_per_step, uint32_t* sink, uint4* out,
                     uint32_t out16, uint32_t out_per_wg16) {
  asm volatile("" ::"s"(p), "s"(bytes), "s"(per_wg), "s"(steps), "s"(slab), "s"(slab_bytes), "s"(slab_groups),
               "s"(slab_per_step));
  asm volatile("" : "+s"(sink), "+s"(out), "+s"(out16), "+s"(out_per_wg16));
  __shared__ uint4 slab_lds[FLOOR_WAVES * WAVE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t grp = (uint32_t)(((uint64_t)blockIdx.x * slab_groups) / gridDim.x);
  const uint32_t slab_loads = (slab_bytes + FLOOR_WAVES * 1024u - 1) / (FLOOR_WAVES * 1024u);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)slab, 0, (int)(slab_bytes * slab_groups), RSRC_WORD3);
  const lds_addr_t dst = lds_addr(slab_lds + wave * WAVE);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)bytes, RSRC_WORD3);
  const uint32_t begin = blockIdx.x * per_wg;
  const uint32_t end = min(begin + per_wg, bytes);
  const uint32_t first = begin + (uint32_t)wave * 1024u + (uint32_t)lane * 16u;
  uint32_t acc = 0;
  for (uint32_t st = 0; st < steps; ++st) {
    const uint32_t i_end = min((st + 1) * slab_per_step, slab_loads);
    for (uint32_t i = st * slab_per_step; i < i_end; ++i) {
      const uint32_t off = ((uint32_t)wave + FLOOR_WAVES * i) * 1024u + (uint32_t)lane * 16u;
      lds_load16(rs, dst, off < slab_bytes ? grp * slab_bytes + off : OOB);
    }
    uint4 v[L];
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const uint32_t off = first + (st * L + (uint32_t)u) * FLOOR_WAVES * 1024u;
      v[u] = load16_stream(r, off < end ? off : OOB);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < L; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (out) {
    const uint32_t b = blockIdx.x * out_per_wg16, e = min(b + out_per_wg16, out16);
    if (out_per_wg16 >= 1024) {
      const u32x4_t a4 = {acc, acc, acc, acc};
      for (uint32_t i = b + threadIdx.x; i < e; i += WAVE * FLOOR_WAVES)
        __builtin_nontemporal_store(a4, reinterpret_cast<u32x4_t*>(out + i));
    } else {
      for (uint32_t i = b + threadIdx.x; i < e; i += WAVE * FLOOR_WAVES) out[i] = make_uint4(acc, acc, acc, acc);
    }
  } else if (acc == FLOOR_MAGIC) {
    sink[blockIdx.x] = acc;
  }
}

typedef void (*FloorFn)(const uint8_t*, uint32_t, uint32_t, uint32_t, const uint8_t*, uint32_t, uint32_t, uint32_t*,
                        uint4*, uint32_t, uint32_t);
const FloorFn kFloor[FLOOR_MAX_L] = {read_floor_kernel<1>, read_floor_kernel<2>,  read_floor_kernel<3>,
                                     read_floor_kernel<4>, read_floor_kernel<5>,  read_floor_kernel<6>,
                                     read_floor_kernel<7>, read_floor_kernel<8>,  read_floor_kernel<9>,
                                     read_floor_kernel<10>, read_floor_kernel<11>, read_floor_kernel<12>};
typedef void (*FloorIlFn)(const uint8_t*, uint32_t, uint32_t, uint32_t, const uint8_t*, uint32_t, uint32_t, uint32_t,
                          uint32_t*, uint4*, uint32_t, uint32_t);
// a share of several steps takes L = 12
const FloorIlFn kFloorIl = read_floor_il_kernel<FLOOR_MAX_L>;

}  // namespace

int launch_read_floor(const void* p, size_t bytes, int nwg, const void* slab, size_t slab_bytes, int slab_groups,
                      int interleave, uint32_t* sink, void* out, size_t out_bytes, hipStream_t stream) {
  // each workgroup's share in whole 16-byte pieces; one wave load covers 1 KB of it, a step of the
  // 8 waves L KB apiece
  const uint32_t per = (uint32_t)((bytes + (size_t)nwg * 16 - 1) / ((size_t)nwg * 16)) * 16u;
  const uint32_t kb = (per + 1023) / 1024;                       // wave loads a share needs
  const uint32_t loads = (kb + FLOOR_WAVES - 1) / FLOOR_WAVES;   // ... per wave
  const int L = loads == 0 ? 1 : loads < (uint32_t)FLOOR_MAX_L ? (int)loads : FLOOR_MAX_L;
  const uint32_t steps = (loads + (uint32_t)L - 1) / (uint32_t)L;
  const uint32_t out16 = (uint32_t)(out_bytes / 16);
  const uint32_t out_per = (out16 + (uint32_t)nwg - 1) / (uint32_t)nwg;
  if (interleave && slab_bytes && steps > 1) {
    // the slab's loads per wave, spread evenly over the steps (with one step the slab goes first
    // either way)
    const uint32_t slab_loads = (uint32_t)((slab_bytes + FLOOR_WAVES * 1024 - 1) / (FLOOR_WAVES * 1024));
    const uint32_t per_step = (slab_loads + steps - 1) / steps;
    hipLaunchKernelGGL(kFloorIl, dim3((unsigned)nwg), dim3(WAVE * FLOOR_WAVES), 0, stream,
                       reinterpret_cast<const uint8_t*>(p), (uint32_t)bytes, per, steps,
                       reinterpret_cast<const uint8_t*>(slab), (uint32_t)slab_bytes, (uint32_t)slab_groups, per_step,
                       sink, out_bytes ? reinterpret_cast<uint4*>(out) : nullptr, out16, out_per);
    return hip_status(hipGetLastError());
  }
  hipLaunchKernelGGL(kFloor[L - 1], dim3((unsigned)nwg), dim3(WAVE * FLOOR_WAVES), 0, stream,
                     reinterpret_cast<const uint8_t*>(p), (uint32_t)bytes, per, steps,
                     reinterpret_cast<const uint8_t*>(slab), (uint32_t)slab_bytes, (uint32_t)slab_groups, sink,
                     out_bytes ? reinterpret_cast<uint4*>(out) : nullptr, out16, out_per);
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
