// Static device scratch for the GEMM entry point that allocates nothing (bsfp8_gemm_no_alloc).
//
// Callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) still need the split-K workspace of the split plans: fp32
// partials of the tile kernel, or the 64-bit exchange slots of the one-pass kernels. This file
// owns one fixed array for them in the library's own device memory; each GPU the library runs on
// holds its own copy (BSFP8_NO_ALLOC_SCRATCH_BYTES bytes, resident until the process ends).
//
// In host code the array's name is only a stand-in for the device symbol, never a device
// address: its per-device address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is passed to kernels and fill launches.
#include <atomic>
#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[BSFP8_NO_ALLOC_SCRATCH_BYTES];

namespace bsfp8 {
namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// Zero-fills n16 16-byte words with vector stores (a kernel rather than hipMemsetAsync, so that a
// captured graph holds an ordinary kernel node).
__global__ void __launch_bounds__(256) clear_kernel(uint4* p, uint32_t n16) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

int scratch_for_stream(hipStream_t stream, void** out) {
  *out = nullptr;
  int dev = 0;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return BSFP8_EHIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return BSFP8_EHIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES) return BSFP8_EHIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      if (hipGetDevice(&cur) != hipSuccess) return BSFP8_EHIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return BSFP8_EHIP;
      const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return BSFP8_EHIP;
      if (err != hipSuccess || !p || (reinterpret_cast<uintptr_t>(p) & 255)) return BSFP8_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BSFP8_OK;
}

int launch_clear(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return BSFP8_OK;
  if ((bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15) || bytes >= ((size_t)1 << 36)) return BSFP8_EINVAL;
  const uint32_t n16 = (uint32_t)(bytes >> 4);
  const uint32_t blocks = std::min<uint32_t>((n16 + 255) / 256, 1024u);
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(p), n16);
  return hip_status(hipGetLastError());
}

}  // namespace bsfp8
