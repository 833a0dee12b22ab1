// Streaming-read probe: the rate at which HBM delivers a plain contiguous read to a simple
// kernel on this device, the practical ceiling beside the vendor peak for the HBM-bound
// attention kernels. A measurement utility (libpagedkv_probe.so), not part of the path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_kv_probe.h"

namespace {

// Grid-stride read of n16 16-byte words. The XOR of everything read is stored only if it hits
// a sentinel, which keeps the loads live without a write per thread.
__global__ void __launch_bounds__(256) read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
#pragma unroll 8
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int pagedkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                                  hipStream_t stream) {
  if (!buf || !sink || grid <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15)) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
