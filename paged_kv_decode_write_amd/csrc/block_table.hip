// Block tables of blocks larger than 16 tokens, seen as tables of 16-token blocks.
//
// A pool of blocks of block_size = 16*k token slots ([NB][16k][Hkv][D]) holds the same bytes
// as a pool of 16-token blocks ([k*NB][16][Hkv][D]): slots of physical block p are 16-token
// blocks k*p .. k*p + k - 1, and a slot number (block * block_size + offset; the pool of
// physical blocks of block_size token slots and the per-sequence block table are those of the
// mini-vLLM README's paged KV-cache paragraph) names the same row in both views. The
// decode kernels are built for 16-token blocks; for larger blocks they read the 16-token view
// through the table this launch writes: entry j of a row is k * T[j / k] + j % k, where T is
// the caller's row. Entries whose id is outside [0, NB) (unused tail entries, which may hold
// -1) become -1, which no kernel reads as a block.
#include "launch.h"

namespace pagedkv {

__global__ void __launch_bounds__(256)
expand_table_kernel(const int32_t* __restrict__ table, int64_t entries, int32_t max_blocks,
                    int32_t sub, int64_t num_blocks, int32_t* __restrict__ out) {
  const int64_t row_out = (int64_t)max_blocks * sub;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < entries;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / row_out;
    const int32_t j = (int32_t)(i - b * row_out);
    const int32_t t = table[b * max_blocks + j / sub];
    out[i] = t >= 0 && t < num_blocks ? t * sub + j % sub : -1;
  }
}

hipError_t launch_expand_table(const int32_t* table, int32_t batch, int32_t max_blocks,
                               int32_t sub, int64_t num_blocks, int32_t* out,
                               hipStream_t stream) {
  const int64_t entries = (int64_t)batch * max_blocks * sub;
  if (entries <= 0) return hipSuccess;
  int64_t grid = (entries + 255) / 256;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(expand_table_kernel, dim3((unsigned)grid), dim3(256), 0, stream, table,
                     entries, max_blocks, sub, num_blocks, out);
  return hipGetLastError();
}

}  // namespace pagedkv
