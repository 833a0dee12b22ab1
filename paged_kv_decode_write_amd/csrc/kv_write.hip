// Slot-mapping KV write: token t's K and V rows go to slot slot_mapping[t] of the paged
// pools ("vLLM-Style Llama Inference Engine with Tensor Parallelism", How it works, step 3;
// the mini-vLLM README's per-sequence write loop into the block pool, here one scatter
// launch for all tokens). A row is num_kv_heads*head_dim bf16 values, contiguous in both
// the input [T][Hkv][D] and the pool [NB][bs][Hkv][D], so slot s's row starts at element
// s*Hkv*D. The copy moves raw 16-byte words: the bits land unchanged.
#include "launch.h"

namespace pagedkv {

__global__ void __launch_bounds__(256)
kv_write_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                const int64_t* __restrict__ slots, int64_t num_tokens,
                uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int64_t num_slots,
                int32_t row_vecs) {
  for (int64_t t = blockIdx.x; t < num_tokens; t += gridDim.x) {
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;  // padding token, or a slot outside the pool
    const uint4* ks = k + t * row_vecs;
    const uint4* vs = v + t * row_vecs;
    uint4* kd = k_cache + s * row_vecs;
    uint4* vd = v_cache + s * row_vecs;
    for (int i = threadIdx.x; i < row_vecs; i += blockDim.x) {
      const uint4 a = ks[i];
      const uint4 b = vs[i];
      kd[i] = a;
      vd[i] = b;
    }
  }
}

hipError_t launch_kv_write(const uint16_t* k, const uint16_t* v, const int64_t* slots,
                           int64_t num_tokens, uint16_t* k_cache, uint16_t* v_cache,
                           int64_t num_slots, int32_t row_elems, hipStream_t stream) {
  const int32_t row_vecs = row_elems / 8;
  int threads = ((row_vecs + 63) / 64) * 64;
  if (threads > 256) threads = 256;
  const int64_t grid = num_tokens < (1 << 20) ? num_tokens : (1 << 20);
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)grid), dim3(threads), 0, stream,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     slots, num_tokens, reinterpret_cast<uint4*>(k_cache),
                     reinterpret_cast<uint4*>(v_cache), num_slots, row_vecs);
  return hipGetLastError();
}

}  // namespace pagedkv
