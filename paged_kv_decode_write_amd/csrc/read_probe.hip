// Streaming-read probe: the rate at which HBM delivers a plain contiguous read to a simple
// kernel on this device, the practical ceiling beside the vendor peak for the HBM-bound
// attention kernels. A measurement utility (libpagedkv_probe.so), not part of the path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_kv_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte words, plain or with the non-temporal (streaming) hint. The
// XOR of everything read is stored only if it hits a sentinel, which keeps the loads live
// without a write per thread.
template <bool NT>
__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
#pragma unroll 8
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Chunked read: workgroup w reads the w-th contiguous chunk, 256 threads x 4 loads per step
// (four 16-byte loads in flight per thread), with the non-temporal hint.
__global__ void __launch_bounds__(256) read_probe_chunked_nt_kernel(const u32x4* __restrict__ p,
                                                                   size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

template <bool NT>
int launch_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                 hipStream_t stream) {
  if (!buf || !sink || grid <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15)) return 1;
  hipLaunchKernelGGL(read_probe_kernel<NT>, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" int pagedkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                                  hipStream_t stream) {
  return launch_probe<false>(buf, bytes, sink, grid, stream);
}

extern "C" int pagedkv_read_probe_nt(const void* buf, size_t bytes, uint32_t* sink,
                                     int32_t grid, hipStream_t stream) {
  return launch_probe<true>(buf, bytes, sink, grid, stream);
}

extern "C" int pagedkv_read_probe_chunked_nt(const void* buf, size_t bytes, uint32_t* sink,
                                             int32_t grid, hipStream_t stream) {
  if (!buf || !sink || grid <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15)) return 1;
  hipLaunchKernelGGL(read_probe_chunked_nt_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
