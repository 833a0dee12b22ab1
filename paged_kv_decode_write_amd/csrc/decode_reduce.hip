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
// More than 128 partitions (and the multi-query key split): one workgroup of 512 threads per
// (sequence, query head), one barrier. Every memory read is
// issued before any of them is needed, and none waits for another: the merge does not read the
// context length, because a partition past the context marks its rows with m = -inf (no keys)
// and its partial outputs are then never used. Each thread folds what it read with the rule
// above, keeping its own reference max, so nothing waits for the global M either:
//   (m1, x1) + (m2, x2) = (m, 2^(m1 - m) x1 + 2^(m2 - m) x2),  m = max(m1, m2).
// Statistics: thread t folds (m_p, l_p) of partitions t, t + 512, ...; the waves combine them
// by shuffles, the workgroup through LDS. Outputs: thread (column d, group g) folds (m_p,
// a_p[d]) of partitions g, g + 512/D, ... (loads coalesced along d, independent across p);
// the groups combine through LDS. The partials are fp32 whatever the formats; the result is
// stored in the output format.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

constexpr int kReduceThreads = 512;

// (m, x) += (m2, x2) under the rule above. m == -inf means no keys (x is then 0, and an x2
// that comes with m2 == -inf is not read: it may be stale workspace).
__device__ __forceinline__ void fold(float& m, float& x, float m2, float x2) {
  const float mn = fmaxf(m, m2);
  const float ref = mn == kNegInf ? 0.f : mn;
  const float y2 = m2 == kNegInf ? 0.f : x2;
  x = fmaf(x, fast_exp2(m - ref), y2 * fast_exp2(m2 - ref));
  m = mn;
}

// SPARSE (the key split of the multi-query kernel): a row whose first slot holds the done
// marker (-inf, -1) was written out directly and is left alone, and partial outputs are read
// only for partitions that saw keys (m > -inf). That costs a second round trip (statistics,
// then outputs) and saves the reads of the many empty partitions that split causal tiles have.

// PER: partitions per column group read in the first pass (a power of two, at most 16; the
// launch picks the smallest that covers nparts when it can). Used for more than 8 partitions.
template <int OT, int PER, bool SPARSE>
__global__ void __launch_bounds__(kReduceThreads)
decode_reduce_kernel(const DecodeArgs a) {
  constexpr int NWV = kReduceThreads / 64;
  __shared__ float red_m[NWV], red_l[NWV];
  __shared__ float part_m[kReduceThreads], part_x[kReduceThreads];

  const int row = blockIdx.x;  // b * Hq + h
  const int D = a.head_dim;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nparts = a.nparts;
  const float* ml = a.ws_ml + (size_t)row * nparts * 2;
  const float* acc = a.ws_acc + (size_t)row * nparts * D;

  const int groups = kReduceThreads / D;  // D in {64, 128}: 8 or 4
  const int d = tid % D, grp = tid / D;
  if constexpr (SPARSE)
    if (ml[1] < 0.f) return;  // done marker (uniform over the workgroup, before the barrier)

  // First pass, all loads issued together: the statistics of partition tid and (m_p, a_p[d])
  // of partitions grp + u * groups, u < PER. Indices past the end are clamped so that every
  // load is unconditional; their values are masked afterwards.
  const int last = nparts - 1;
  const int ps = tid < nparts ? tid : last;
  const float m_s = ml[2 * ps], l_s = ml[2 * ps + 1];
  float mp[PER], ap[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = grp + u * groups;
    const int pc = p < nparts ? p : last;
    mp[u] = ml[2 * pc];
    if constexpr (!SPARSE) ap[u] = acc[(size_t)pc * D + d];
  }
  if constexpr (SPARSE) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int p = grp + u * groups;
      ap[u] = p < nparts && mp[u] != kNegInf ? acc[(size_t)p * D + d] : 0.f;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads above ahead of every use
  float m = tid < nparts ? m_s : kNegInf, l = tid < nparts ? l_s : 0.f;
  float mx = kNegInf, x = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    fold(mx, x, grp + u * groups < nparts ? mp[u] : kNegInf, ap[u]);
  // The rest, for more than 512 partitions or more than PER per column group.
  for (int p = tid + kReduceThreads; p < nparts; p += kReduceThreads)
    fold(m, l, ml[2 * p], ml[2 * p + 1]);
  for (int p = grp + PER * groups; p < nparts; p += groups) {
    const float m2 = ml[2 * p];
    fold(mx, x, m2, !SPARSE || m2 != kNegInf ? acc[(size_t)p * D + d] : 0.f);
  }

#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float m2 = shfl_xor(m, s), l2 = shfl_xor(l, s);
    fold(m, l, m2, l2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_l[wave] = l;
  }
  part_m[tid] = mx;
  part_x[tid] = x;
  __syncthreads();
  if (grp != 0) return;
  float M = red_m[0], den = red_l[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) fold(M, den, red_m[w], red_l[w]);
  float mo = part_m[d], num = part_x[d];
  for (int q = 1; q < groups; ++q) fold(mo, num, part_m[q * D + d], part_x[q * D + d]);
  // num and den end on the same reference: mo and M are maxima of the same set of m_p.
  store_out<OT>(a.out, (size_t)row * D + d, den > 0.f ? num / den : 0.f);
}

// Few partitions (nparts <= NP <= 8): one thread per four consecutive output elements reads
// the statistics and its four columns of every partition at once (16-byte loads) and folds
// them in partition order; no LDS, no barrier. The statistics are the same few addresses for
// the D/4 threads of a row. The sum and the four outputs share one reference max, so the
// weights 2^(m - ref) and 2^(m_p - ref) are computed once per partition for all five.
constexpr int kNarrowThreads = 256;

template <int OT, int NP, bool SPARSE>
__global__ void __launch_bounds__(kNarrowThreads)
decode_reduce_narrow_kernel(const DecodeArgs a) {
  const int D = a.head_dim;  // 64 or 128: a workgroup covers 4 * kNarrowThreads / D rows
  const int tpr = D / 4;     // threads per row
  const size_t row = (size_t)blockIdx.x * (kNarrowThreads / tpr) + threadIdx.x / tpr;
  const int d = 4 * (threadIdx.x % tpr);
  if (row >= (size_t)a.batch * a.num_q_heads) return;
  const int nparts = a.nparts, last = nparts - 1;
  const float* ml = a.ws_ml + row * nparts * 2;
  const float* acc = a.ws_acc + row * nparts * D + d;
  float mp[NP], lp[NP];
  float4 ap[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pc = u < nparts ? u : last;
    mp[u] = ml[2 * pc];
    lp[u] = ml[2 * pc + 1];
    if constexpr (!SPARSE) ap[u] = *reinterpret_cast<const float4*>(acc + (size_t)pc * D);
  }
  if constexpr (SPARSE) {
    if (lp[0] < 0.f) return;  // done marker: written out directly
#pragma unroll
    for (int u = 0; u < NP; ++u)
      ap[u] = u < nparts && mp[u] != kNegInf
                  ? *reinterpret_cast<const float4*>(acc + (size_t)u * D)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads above ahead of every use
  // fold() of (m, l) and of (m, a[k]) for k < 4, which see the same maxima
  float m = kNegInf, l = 0.f;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const float m2 = u < nparts ? mp[u] : kNegInf;
    const float mn = fmaxf(m, m2);
    const float ref = mn == kNegInf ? 0.f : mn;
    const bool none = m2 == kNegInf;
    const float s1 = fast_exp2(m - ref), s2 = fast_exp2(m2 - ref);
    l = fmaf(l, s1, (none ? 0.f : lp[u]) * s2);
    x.x = fmaf(x.x, s1, (none ? 0.f : ap[u].x) * s2);
    x.y = fmaf(x.y, s1, (none ? 0.f : ap[u].y) * s2);
    x.z = fmaf(x.z, s1, (none ? 0.f : ap[u].z) * s2);
    x.w = fmaf(x.w, s1, (none ? 0.f : ap[u].w) * s2);
    m = mn;
  }
  store_out4<OT>(a.out, row * D + d, l > 0.f ? x.x / l : 0.f, l > 0.f ? x.y / l : 0.f,
                 l > 0.f ? x.z / l : 0.f, l > 0.f ? x.w / l : 0.f);
}

// Up to 128 partitions: SPLIT consecutive lanes share four consecutive output columns of a row
// and split its partitions between them, lane j reading partitions j, j + SPLIT, ... (NP of
// them, clamped and masked past the end). Every lane issues all its loads at once (16-byte
// partial outputs, 8-byte statistics), folds them in partition order as the narrow form does,
// and the SPLIT lanes then combine their (max, sum, four outputs) by shuffles. No LDS and no
// barrier: the whole merge is one round trip to memory plus log2(SPLIT) shuffle steps.
// LIVE: read a slot's partial output only when its statistics say it saw keys (m > -inf): a
// second round trip, worth it when most slots are empty (the stream family's, whose slot count
// bounds the segments a sequence can need while a uniform batch uses a few of them).
template <int OT, int NP, int SPLIT, bool LIVE>
__global__ void __launch_bounds__(256)
decode_reduce_split_kernel(const DecodeArgs a) {
  const int D = a.head_dim;
  const int tpr = (D / 4) * SPLIT;  // threads per row
  const size_t row = (size_t)blockIdx.x * (blockDim.x / tpr) + threadIdx.x / tpr;
  const int j = threadIdx.x % SPLIT;
  const int d = 4 * ((threadIdx.x % tpr) / SPLIT);
  const bool live = row < (size_t)a.batch * a.num_q_heads;
  const size_t r = live ? row : 0;  // dead lanes load row 0 and store nothing
  const int nparts = a.nparts, last = nparts - 1;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + r * nparts;
  const float* acc = a.ws_acc + r * nparts * D + d;
  float2 st[NP];
  float4 ap[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = j + u * SPLIT;
    const int pc = p < nparts ? p : last;
    st[u] = ml[pc];
    if constexpr (!LIVE) ap[u] = *reinterpret_cast<const float4*>(acc + (size_t)pc * D);
  }
  if constexpr (LIVE)  // with the statistics: slot j (see below)
    ap[0] = *reinterpret_cast<const float4*>(acc + (size_t)(j < nparts ? j : last) * D);
  if constexpr (LIVE) {
    // The first SPLIT slots were read with the statistics (a sequence's first segments fill the
    // lowest slots, so on a uniform batch these are all its live ones); the rest only if live.
#pragma unroll
    for (int u = 1; u < NP; ++u) {
      const int p = j + u * SPLIT;
      ap[u] = p < nparts && st[u].x != kNegInf
                  ? *reinterpret_cast<const float4*>(acc + (size_t)p * D)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads above ahead of every use
  float m = kNegInf, l = 0.f;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const float m2 = j + u * SPLIT < nparts ? st[u].x : kNegInf;
    const float mn = fmaxf(m, m2);
    const float ref = mn == kNegInf ? 0.f : mn;
    const bool none = m2 == kNegInf;
    const float s1 = fast_exp2(m - ref), s2 = fast_exp2(m2 - ref);
    l = fmaf(l, s1, (none ? 0.f : st[u].y) * s2);
    x.x = fmaf(x.x, s1, (none ? 0.f : ap[u].x) * s2);
    x.y = fmaf(x.y, s1, (none ? 0.f : ap[u].y) * s2);
    x.z = fmaf(x.z, s1, (none ? 0.f : ap[u].z) * s2);
    x.w = fmaf(x.w, s1, (none ? 0.f : ap[u].w) * s2);
    m = mn;
  }
#pragma unroll
  for (int s = 1; s < SPLIT; s <<= 1) {
    const float m2 = shfl_xor(m, s), l2 = shfl_xor(l, s);
    const float x0 = shfl_xor(x.x, s), x1 = shfl_xor(x.y, s), x2 = shfl_xor(x.z, s),
                x3 = shfl_xor(x.w, s);
    const float mn = fmaxf(m, m2);
    const float ref = mn == kNegInf ? 0.f : mn;
    const float s1 = fast_exp2(m - ref), s2 = fast_exp2(m2 - ref);
    l = fmaf(l, s1, l2 * s2);
    x.x = fmaf(x.x, s1, x0 * s2);
    x.y = fmaf(x.y, s1, x1 * s2);
    x.z = fmaf(x.z, s1, x2 * s2);
    x.w = fmaf(x.w, s1, x3 * s2);
    m = mn;
  }
  if (live && j == 0)
    store_out4<OT>(a.out, row * D + d, l > 0.f ? x.x / l : 0.f, l > 0.f ? x.y / l : 0.f,
                   l > 0.f ? x.z / l : 0.f, l > 0.f ? x.w / l : 0.f);
}

template <int OT, int NP, int SPLIT>
hipError_t launch_split_merge(const DecodeArgs& a, unsigned rows, hipStream_t stream) {
  const int tpr = (a.head_dim / 4) * SPLIT;
  const int block = tpr >= 128 ? tpr : 128;
  const unsigned per = (unsigned)(block / tpr);
  if (a.sk_min_pairs > 0)  // the stream family's slots: mostly empty on uniform batches
    hipLaunchKernelGGL((decode_reduce_split_kernel<OT, NP, SPLIT, true>),
                       dim3((rows + per - 1) / per), dim3(block), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_split_kernel<OT, NP, SPLIT, false>),
                       dim3((rows + per - 1) / per), dim3(block), 0, stream, a);
  return hipGetLastError();
}

template <int OT, bool SPARSE>
hipError_t launch_reduce_per(const DecodeArgs& a, unsigned rows, hipStream_t stream) {
  if (a.nparts <= 8) {
    const unsigned grid =
        (unsigned)(((size_t)rows * (a.head_dim / 4) + kNarrowThreads - 1) / kNarrowThreads);
    const dim3 block(kNarrowThreads);
    if (a.nparts <= 2)
      hipLaunchKernelGGL((decode_reduce_narrow_kernel<OT, 2, SPARSE>), dim3(grid), block, 0,
                         stream, a);
    else if (a.nparts <= 4)
      hipLaunchKernelGGL((decode_reduce_narrow_kernel<OT, 4, SPARSE>), dim3(grid), block, 0,
                         stream, a);
    else
      hipLaunchKernelGGL((decode_reduce_narrow_kernel<OT, 8, SPARSE>), dim3(grid), block, 0,
                         stream, a);
    return hipGetLastError();
  }
  if constexpr (!SPARSE) {
    if (a.nparts <= 16) return launch_split_merge<OT, 4, 4>(a, rows, stream);
    if (a.nparts <= 32) return launch_split_merge<OT, 8, 4>(a, rows, stream);
    if (a.nparts <= 64) return launch_split_merge<OT, 16, 4>(a, rows, stream);
    if (a.nparts <= 128) return launch_split_merge<OT, 16, 8>(a, rows, stream);
  }
  const int groups = kReduceThreads / a.head_dim;
  const int need = (a.nparts + groups - 1) / groups;
  const dim3 grid(rows), block(kReduceThreads);
  if (need <= 1)
    hipLaunchKernelGGL((decode_reduce_kernel<OT, 1, SPARSE>), grid, block, 0, stream, a);
  else if (need <= 2)
    hipLaunchKernelGGL((decode_reduce_kernel<OT, 2, SPARSE>), grid, block, 0, stream, a);
  else if (need <= 4)
    hipLaunchKernelGGL((decode_reduce_kernel<OT, 4, SPARSE>), grid, block, 0, stream, a);
  else if (need <= 8)
    hipLaunchKernelGGL((decode_reduce_kernel<OT, 8, SPARSE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<OT, 16, SPARSE>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <bool SPARSE>
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)((long long)a.batch * a.num_q_heads);
  switch (a.out_dtype) {
    case kDtF32: return launch_reduce_per<kDtF32, SPARSE>(a, rows, stream);
    case kDtBf16: return launch_reduce_per<kDtBf16, SPARSE>(a, rows, stream);
    case kDtF16: return launch_reduce_per<kDtF16, SPARSE>(a, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  return launch_reduce<false>(a, stream);
}

hipError_t launch_prefill_merge(const DecodeArgs& a, hipStream_t stream) {
  return launch_reduce<true>(a, stream);
}

}  // namespace pagedkv
