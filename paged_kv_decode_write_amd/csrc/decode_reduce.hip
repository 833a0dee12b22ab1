// Merge of per-partition partial softmax results (split-K / flash-decoding).
//
// A partition p of a sequence's keys leaves, per query head, its running max m_p, the sum
// l_p = sum_t 2^(s_t - m_p) and the unnormalised output a_p = sum_t 2^(s_t - m_p) v_t, with
// scores s in log2 units. The exact softmax output over all keys is
//   out = sum_p 2^(m_p - M) a_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// the running-max rescaling of the tiled online softmax (llm-stack, Attention kernel
// section) applied across partitions instead of across tiles. The long-context decode page
// that motivates the split lists a split-K kernel as out of its scope ("vLLM-Style Llama
// Inference Engine with Tensor Parallelism", Out of scope); this is the merge it would need.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

// One workgroup per (sequence, query head); thread d owns output column d (blockDim = D).
__global__ void __launch_bounds__(128)
decode_reduce_kernel(const DecodeArgs a) {
  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / a.num_q_heads;
  const int D = a.head_dim;
  const int d = threadIdx.x;
  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * a.block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  float* o = a.out + (size_t)row * D;
  if (L == 0) {
    if (d < D) o[d] = 0.f;
    return;
  }
  const int np = (L + a.part_tokens - 1) / a.part_tokens;  // partitions holding keys
  const float* ml = a.ws_ml + (size_t)row * a.nparts * 2;
  const float* acc = a.ws_acc + (size_t)row * a.nparts * D;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  float num = 0.f, den = 0.f;
  if (M != kNegInf) {
    for (int p = 0; p < np; ++p) {
      const float f = fast_exp2(ml[2 * p] - M);
      den = fmaf(f, ml[2 * p + 1], den);
      if (d < D) num = fmaf(f, acc[(size_t)p * D + d], num);
    }
  }
  if (d < D) o[d] = den > 0.f ? num / den : 0.f;
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.batch * a.num_q_heads;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)rows), dim3(a.head_dim), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace pagedkv
