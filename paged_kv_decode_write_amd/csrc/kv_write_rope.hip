// Rotary position embedding at absolute positions fused with the slot-mapping KV write.
//
// Keys must be rotated at their absolute positions before they enter the cache (llm-stack,
// Serving engine / KV cache bullet); the rotation turns pairs of components of each head
// vector by position-dependent angles with sine and cosine ("tiny-vLLM" blog, CUDA Kernel
// Engineering: RoPE). For token t at position p and pair i: theta = p * inv_freq[i] (fp32),
// (x0, x1) -> (x0 cos - x1 sin, x1 cos + x0 sin), pairs (i, i + D/2) or (2i, 2i+1). q is
// rotated into q_out; k is rotated and stored, v copied, at slot slot_mapping[t] (as the
// plain write does; a negative slot stores nothing). One launch does what would otherwise be
// a rotation kernel, a write kernel and a second pass over k.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// One workgroup per token. Thread (pair i, slice j) forms the angle of pair i and its sine
// and cosine once, then rotates pair i of heads j, j + NS, j + 2*NS, ... of q and of k
// (NS = 256 / (D/2) slices), so the transcendental work is NS per pair rather than one per
// head, while every thread still has only a few heads to rotate.
__device__ __forceinline__ void rotate_pair(const uint16_t* src, uint16_t* dst, int i0, int i1,
                                            float cs, float sn) {
  float y0, y1;
  rope_rotate(bf16_to_f32(src[i0]), bf16_to_f32(src[i1]), cs, sn, y0, y1);
  dst[i0] = f32_to_bf16_rne(y0);
  dst[i1] = f32_to_bf16_rne(y1);
}

__global__ void __launch_bounds__(256)
kv_write_rope_kernel(const RopeArgs a) {
  const int D = a.head_dim, half = D / 2;
  const int NS = 256 / half;
  const int i = threadIdx.x % half;
  const int slice = threadIdx.x / half;
  const int i0 = a.interleaved ? 2 * i : i;
  const int i1 = a.interleaved ? 2 * i + 1 : i + half;
  for (int64_t t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
    if (slice >= NS) break;  // only when 256 is not a multiple of D/2
    float sn, cs;
    sincosf((float)a.positions[t] * a.inv_freq[i], &sn, &cs);
    const uint16_t* qs = a.q + (size_t)t * a.num_q_heads * D;
    uint16_t* qd = a.q_out + (size_t)t * a.num_q_heads * D;
    for (int h = slice; h < a.num_q_heads; h += NS) rotate_pair(qs + h * D, qd + h * D, i0, i1, cs, sn);
    const int64_t s = a.slot_mapping[t];
    if (s >= 0 && s < a.num_slots) {
      const uint16_t* ks = a.k + (size_t)t * a.num_kv_heads * D;
      uint16_t* kd = a.k_cache + (size_t)s * a.num_kv_heads * D;
      for (int h = slice; h < a.num_kv_heads; h += NS)
        rotate_pair(ks + h * D, kd + h * D, i0, i1, cs, sn);
      // v: raw copy of the token's row, 16 bytes per thread and step
      const int row_vecs = a.num_kv_heads * D / 8;
      const uint4* vs = reinterpret_cast<const uint4*>(a.v) + t * row_vecs;
      uint4* vd = reinterpret_cast<uint4*>(a.v_cache) + s * row_vecs;
      for (int x = threadIdx.x; x < row_vecs; x += 256) vd[x] = vs[x];
    }
  }
}

hipError_t launch_kv_write_rope(const RopeArgs& a, hipStream_t stream) {
  const int64_t grid = a.num_tokens < (1 << 20) ? a.num_tokens : (1 << 20);
  hipLaunchKernelGGL(kv_write_rope_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pagedkv
