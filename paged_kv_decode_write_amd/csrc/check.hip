// Device-side validation of the data a call reads, for the checked build (PAGEDKV_CHECKED).
//
// The library's contract leaves data-dependent validity to the caller: slot ids inside the
// pool, block ids inside the pool for every block a context covers, lengths within the table
// width, query spans that fit their contexts. Checking them on the host would need a copy
// back and a synchronisation, so the kernels only stay memory-safe on bad data (they skip or
// clamp) and the answer is then silently wrong. A paged kernel's result is defined by the
// dense attention over the blocks its table names (mini-vLLM README, paged KV-cache paragraph
// and its test of the paged kernel against dense attention on scattered blocks); the checked
// build makes a violation of that contract visible. Before a call's kernels, it launches these
// checks on the same stream; the first violation found is recorded in a per-device error
// record, which paged_kv_check_status reads after a synchronisation. The unchecked library
// compiles the same kernels but never launches them.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace pagedkv {

namespace {

// [0] code (0: none), [1] index, [2] value. Zero when the code object loads.
__device__ unsigned long long g_check[3];

// Records a violation unless one is already recorded. Only the lane whose compare-and-swap
// finds the record empty writes the index and value; every access is a per-lane (vector)
// global memory operation.
__device__ __forceinline__ void record(int code, long long index, long long value) {
  if (atomicCAS(&g_check[0], 0ull, (unsigned long long)code) == 0ull) {
    __hip_atomic_store(&g_check[1], (unsigned long long)index, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g_check[2], (unsigned long long)value, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Slot ids: negative means padding (no write); otherwise below num_slots.
__global__ void check_slots_kernel(const int64_t* __restrict__ slots, int64_t n,
                                   int64_t num_slots) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = slots[t];
    if (s >= num_slots) record(kCheckSlot, t, s);
  }
}

// One workgroup per sequence: 0 <= context_lens[b] <= max_blocks * block_size, and every table
// entry the context covers (the first ceil(L / block_size)) names a block of the pool.
__global__ void check_tables_kernel(const int32_t* __restrict__ tables,
                                    const int32_t* __restrict__ lens, int32_t max_blocks,
                                    int32_t block_size, int64_t num_blocks) {
  const int b = blockIdx.x;
  int L = lens[b];
  const int64_t Lmax = (int64_t)max_blocks * block_size;
  if (L < 0 || L > Lmax) {
    if (threadIdx.x == 0) record(kCheckLength, b, L);
    L = L < 0 ? 0 : (int)Lmax;
  }
  const int nblk = (int)(((int64_t)L + block_size - 1) / block_size);
  const int32_t* row = tables + (size_t)b * max_blocks;
  for (int j = threadIdx.x; j < nblk; j += blockDim.x) {
    const int32_t id = row[j];
    if (id < 0 || (int64_t)id >= num_blocks) record(kCheckBlock, (int64_t)b * max_blocks + j, id);
  }
}

// Query spans of the multi-query call: cu_seqlens_q non-decreasing from 0 <= cu[0] to
// cu[B] <= num_tokens, and each sequence's span Q_b no longer than its context (its rows are
// its last Q_b positions) nor than max_q_len (which sizes the grid).
__global__ void check_queries_kernel(const int32_t* __restrict__ cu,
                                     const int32_t* __restrict__ lens, int32_t batch,
                                     int32_t max_blocks, int32_t block_size,
                                     int64_t num_tokens, int32_t max_q_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int q0 = cu[b], q1 = cu[b + 1];
  if (q0 < 0 || q1 < q0 || q1 > num_tokens) {
    record(kCheckQuery, b, (int64_t)q1 - q0);
    return;
  }
  int64_t L = lens[b];
  const int64_t Lmax = (int64_t)max_blocks * block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  if (q1 - q0 > L || q1 - q0 > max_q_len) record(kCheckQuery, b, q1 - q0);
}

}  // namespace

hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t num_slots,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, stream, slots, n, num_slots);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* tables, const int32_t* lens, int32_t batch,
                               int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_tables_kernel, dim3(batch), dim3(256), 0, stream, tables, lens,
                     max_blocks, block_size, num_blocks);
  return hipGetLastError();
}

hipError_t launch_check_queries(const int32_t* cu, const int32_t* lens, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int64_t num_tokens,
                                int32_t max_q_len, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_queries_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, cu,
                     lens, batch, max_blocks, block_size, num_tokens, max_q_len);
  return hipGetLastError();
}

hipError_t read_check_record(long long rec[3], bool clear) {
  unsigned long long h[3] = {0, 0, 0};
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_check), sizeof h, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (int i = 0; i < 3; ++i) rec[i] = (long long)h[i];
  if (clear) {
    const unsigned long long z[3] = {0, 0, 0};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_check), z, sizeof z, 0, hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace pagedkv
