// Merge of per-partition partial softmax results (split-K / flash-decoding).
//
// A partition p of a sequence's keys leaves, per query head, a reference max m_p (log2
// units), the sum l_p = sum_t 2^(s_t - m_p) and the unnormalised output
// a_p = sum_t 2^(s_t - m_p) v_t. The exact softmax output over all keys is
//   out = sum_p 2^(m_p - M) a_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// the running-max rescaling of the tiled online softmax (llm-stack, Attention kernel
// section) applied across partitions instead of across tiles. The long-context decode page
// that motivates the split lists a split-K kernel as out of its scope ("vLLM-Style Llama
// Inference Engine with Tensor Parallelism", Out of scope); this is the merge it would need.
//
// One workgroup of 256 threads per (sequence, query head). The partition statistics are
// reduced across the whole workgroup; the weighted sum of the partial outputs splits the
// partitions over 256/D thread groups (thread = (column d, group)), whose loads of a_p are
// coalesced along d and independent across p. The partials are fp32 whatever the formats;
// the result is stored in the output format.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

constexpr int kReduceThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) v = fmaxf(v, shfl_xor(v, x));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) v += shfl_xor(v, x);
  return v;
}

template <int OT>
__global__ void __launch_bounds__(kReduceThreads)
decode_reduce_kernel(const DecodeArgs a) {
  constexpr int NWV = kReduceThreads / 64;
  __shared__ float red[NWV];
  __shared__ float part[kReduceThreads];

  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / a.num_q_heads;
  const int D = a.head_dim;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * a.block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const size_t o = (size_t)row * D;
  if (L == 0) {
    for (int d = tid; d < D; d += kReduceThreads) store_out<OT>(a.out, o + d, 0.f);
    return;
  }
  const int np = (L + a.part_tokens - 1) / a.part_tokens;  // partitions holding keys
  const float* ml = a.ws_ml + (size_t)row * a.nparts * 2;
  const float* acc = a.ws_acc + (size_t)row * a.nparts * D;

  // M = max_p m_p over the workgroup.
  float M = kNegInf;
  for (int p = tid; p < np; p += kReduceThreads) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  // den = sum_p 2^(m_p - M) l_p.
  float den = 0.f;
  if (M != kNegInf)
    for (int p = tid; p < np; p += kReduceThreads)
      den = fmaf(fast_exp2(ml[2 * p] - M), ml[2 * p + 1], den);
  den = wave_sum(den);
  if (lane == 0) red[wave] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) den += red[w];

  // num[d] = sum_p 2^(m_p - M) a_p[d], partitions split over `groups` thread groups.
  const int groups = kReduceThreads / D;  // D in {64, 128}: 4 or 2
  const int d = tid % D, grp = tid / D;
  float num = 0.f;
  if (M != kNegInf) {
#pragma unroll 4
    for (int p = grp; p < np; p += groups)
      num = fmaf(fast_exp2(ml[2 * p] - M), acc[(size_t)p * D + d], num);
  }
  part[tid] = num;
  __syncthreads();
  if (grp == 0) {
    for (int q = 1; q < groups; ++q) num += part[q * D + d];
    store_out<OT>(a.out, o + d, den > 0.f ? num / den : 0.f);
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)((long long)a.batch * a.num_q_heads);
  switch (a.out_dtype) {
    case kDtF32: hipLaunchKernelGGL(decode_reduce_kernel<kDtF32>, dim3(rows), dim3(kReduceThreads), 0, stream, a); break;
    case kDtBf16: hipLaunchKernelGGL(decode_reduce_kernel<kDtBf16>, dim3(rows), dim3(kReduceThreads), 0, stream, a); break;
    case kDtF16: hipLaunchKernelGGL(decode_reduce_kernel<kDtF16>, dim3(rows), dim3(kReduceThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pagedkv
