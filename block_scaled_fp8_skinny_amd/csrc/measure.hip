// Measurement aid: the plain-read floor of a weight stream on gfx950.
//
// The GEMM's cost at decode row counts is the time to stream its weight bytes from HBM plus a
// fixed launch and first-byte latency. This kernel does only the first part of that work: it
// reads `bytes` of a buffer once, with the GEMM's load shape (16 bytes per lane, one contiguous
// kilobyte per wave load, non-temporal, several loads in flight per wave), and folds what it read
// into one word per lane, which it stores only if it matches a constant no realistic data hits
// (the store keeps the loads alive; the sink is written at most once per workgroup in practice).
// Timed on the same distinct weight copies as the GEMM, it is the floor a GEMM of that size can
// approach on this machine; with bytes = 0 it is the cost of a launch. With an output buffer it
// also writes `out_bytes` there (16 bytes per lane, each workgroup one contiguous share, after
// its reads): the read + write floor of a GEMM that streams those bytes and stores that many
// output bytes (a kernel that stores pays for its writes and their completion at its end).
#include "device.h"

namespace bsfp8 {
namespace {

constexpr int FLOOR_WAVES = 8;
constexpr int FLOOR_INFLIGHT = 8;                   // loads in flight per wave per step
constexpr uint32_t FLOOR_MAGIC = 0x9E3779B9u;

__global__ void __launch_bounds__(WAVE * FLOOR_WAVES)
read_floor_kernel(const uint8_t* p, uint32_t bytes, uint32_t per_wg, uint32_t* sink, uint4* out, uint32_t out16,
                  uint32_t out_per_wg16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)bytes, RSRC_WORD3);
  const uint32_t begin = blockIdx.x * per_wg;
  const uint32_t end = min(begin + per_wg, bytes);
  uint32_t acc = 0;
  for (uint32_t base = begin + (uint32_t)wave * 1024u; base < end;
       base += (uint32_t)(FLOOR_WAVES * FLOOR_INFLIGHT) * 1024u) {
    uint4 v[FLOOR_INFLIGHT];
#pragma unroll
    for (int u = 0; u < FLOOR_INFLIGHT; ++u) {
      const uint32_t off = base + (uint32_t)u * FLOOR_WAVES * 1024u + (uint32_t)lane * 16u;
      v[u] = load16_stream(r, off < end ? off : OOB);
    }
#pragma unroll
    for (int u = 0; u < FLOOR_INFLIGHT; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (out) {
    const uint32_t b = blockIdx.x * out_per_wg16, e = min(b + out_per_wg16, out16);
    for (uint32_t i = b + threadIdx.x; i < e; i += WAVE * FLOOR_WAVES) out[i] = make_uint4(acc, acc, acc, acc);
  } else if (acc == FLOOR_MAGIC) {
    sink[blockIdx.x] = acc;
  }
}

}  // namespace

int launch_read_floor(const void* p, size_t bytes, int nwg, uint32_t* sink, void* out, size_t out_bytes,
                      hipStream_t stream) {
  const uint32_t per = (uint32_t)((bytes + (size_t)nwg * 1024 - 1) / ((size_t)nwg * 1024)) * 1024u;
  const uint32_t out16 = (uint32_t)(out_bytes / 16);
  const uint32_t out_per = (out16 + (uint32_t)nwg - 1) / (uint32_t)nwg;
  hipLaunchKernelGGL(read_floor_kernel, dim3((unsigned)nwg), dim3(WAVE * FLOOR_WAVES), 0, stream,
                     reinterpret_cast<const uint8_t*>(p), (uint32_t)bytes, per, sink,
                     out_bytes ? reinterpret_cast<uint4*>(out) : nullptr, out16, out_per);
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
