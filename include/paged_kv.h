/*
 * paged_kv.h -- C ABI of libpagedkv: paged KV-cache decode attention and the slot-mapping
 * KV write, for AMD Instinct MI355X (gfx950).
 *
 * The problem these calls solve is the one stated by the pages this library follows:
 *   - "vLLM-Style Llama Inference Engine with Tensor Parallelism", Features and scope /
 *     Implemented: paged KV caching with block tables and slot mappings, grouped-query
 *     attention, and a custom kernel for one-token paged decode attention; How it works,
 *     steps 3-4: each rank writes new K/V into its paged cache, then one-token decode runs a
 *     paged attention kernel.
 *   - mini-vLLM LLM-Inference-Engine README, paged KV-cache paragraph: a fixed pool of
 *     physical blocks, each holding block_size token slots, and a per-sequence block table
 *     that maps logical positions to physical blocks.
 *   - "tiny-vLLM" blog, Mastering the Hardware: allocate device memory once and reuse it.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers to row-major, contiguous arrays, 16-byte
 *     aligned. bf16 values are passed as their uint16_t bit patterns.
 *   - The caller owns every buffer (inputs, outputs, workspace). The library allocates and
 *     frees nothing during a call and keeps no pointer after it returns. Its only state is
 *     a per-device cache of device properties (compute-unit count), filled on first use, and
 *     the static scratch array of paged_decode_step_noalloc (one per device).
 *   - Calls are asynchronous: kernels are enqueued on `stream` (NULL = the null stream) and
 *     the call returns without synchronising. Ordering between a write and a later
 *     attention call is the caller's stream order.
 *   - Calls return a pagedkv_status and never throw. Argument errors are detected on the
 *     host before anything is enqueued. Data-dependent validity (slot ids, block ids,
 *     context lengths) is the caller's contract and is not checked on the host, because
 *     that would need a device-to-host copy; the kernels stay memory-safe on invalid data
 *     (out-of-range slots are not written, out-of-range block ids are not read, lengths are
 *     clamped to the table width) but the results for such entries are unspecified. The
 *     checked build of the library (libpagedkv_checked.so, compiled with PAGEDKV_CHECKED)
 *     validates that data on the device before each call's kernels and records the first
 *     violation for paged_kv_check_status.
 *
 * Cache layout (both pools): [num_blocks][block_size][num_kv_heads][head_dim], 16-bit
 * elements (bf16, or fp16 where a call takes a pagedkv_dtype).
 * Logical position t of a sequence with table row T lives in block T[t / block_size] at
 * offset t % block_size; the slot number of (block, offset) is block*block_size + offset.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGED_KV_ABI_VERSION 6

typedef enum {
  PAGEDKV_OK = 0,
  PAGEDKV_ERR_NULL = 1,        /* a required pointer is NULL */
  PAGEDKV_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent */
  PAGEDKV_ERR_UNSUPPORTED = 3, /* head_dim / block_size / group size / kernel not built */
  PAGEDKV_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  PAGEDKV_ERR_HIP = 5,         /* a HIP runtime call failed; see paged_kv_last_error() */
  PAGEDKV_ERR_ALIGN = 6        /* an array pointer is not 16-byte aligned */
} pagedkv_status;

/*
 * Element formats of the attention inputs and outputs. q and both caches share one 16-bit
 * format: bf16 (8 exponent bits, 7 fraction bits) or fp16 (IEEE binary16: 5 and 10), the two
 * half-width formats the pages weigh against each other ("tiny-vLLM" blog, The Precision
 * Trade-off: BF16; the mini-vLLM README's Results were measured with an fp16 model). The
 * output is fp32, or the input format itself, rounded to nearest even, for a consumer that
 * takes the attention output as the next matrix product's 16-bit operand.
 */
typedef enum {
  PAGEDKV_DTYPE_BF16 = 0,
  PAGEDKV_DTYPE_F16 = 1,
  PAGEDKV_DTYPE_F32 = 2
} pagedkv_dtype;

/* Returns PAGED_KV_ABI_VERSION of the built library. */
int paged_kv_abi_version(void);

/* Static, NUL-terminated name of a status code ("PAGEDKV_OK", ...); never NULL. */
const char* paged_kv_status_string(int status);

/* Text of the last error raised on the calling thread (argument problem or HIP error
 * string); "" if none. Valid until the thread's next call into the library. */
const char* paged_kv_last_error(void);

/*
 * Checked build. A paged kernel's result is defined by the dense attention over the blocks
 * its table names (the mini-vLLM README tests its paged kernel against dense attention on
 * scattered blocks), so a wrong slot or block id or length silently changes the answer. In a
 * library built with PAGEDKV_CHECKED, every call first launches, on its own stream, kernels
 * that validate the data it is about to read: slot ids (below num_blocks * block_size, or
 * negative for padding), context lengths (0 .. max_blocks_per_seq * block_size), the block
 * ids each context covers (the first ceil(L / block_size) table entries, in [0, num_blocks)),
 * and for the multi-query calls the query spans. The first violation found on a device is kept
 * in a per-device record until cleared; the calls themselves then proceed as in the unchecked
 * build (memory-safe, result unspecified).
 */
typedef enum {
  PAGEDKV_CHECK_NONE = 0,
  PAGEDKV_CHECK_SLOT = 1,   /* index: token t; value: slot_mapping[t] >= num_blocks * block_size */
  PAGEDKV_CHECK_LENGTH = 2, /* index: sequence b; value: context_lens[b] < 0 or past the table */
  PAGEDKV_CHECK_BLOCK = 3,  /* index: b * max_blocks_per_seq + j; value: the block id outside
                               [0, num_blocks) of table entry j < ceil(L_b / block_size) */
  PAGEDKV_CHECK_QUERY = 4   /* index: sequence b; value: its span cu[b + 1] - cu[b], which is
                               negative, reaches past num_tokens, or exceeds L_b or max_q_len */
} pagedkv_check_code;

/* 1 if this library was built with PAGEDKV_CHECKED, else 0. Host only. */
int paged_kv_checked_build(void);

/*
 * Synchronises the current device (hipDeviceSynchronize), then reads its check record:
 * *code a pagedkv_check_code (PAGEDKV_CHECK_NONE if no violation was recorded since the last
 * clear), *index and *value (either may be NULL) as listed above. clear != 0 resets the record
 * afterwards. Which of several concurrent violations is recorded is unspecified.
 * Errors: PAGEDKV_ERR_UNSUPPORTED in the unchecked build; PAGEDKV_ERR_NULL for a NULL code;
 * PAGEDKV_ERR_HIP if the synchronisation or the copy fails (including an earlier kernel fault).
 */
int paged_kv_check_status(int32_t* code, int64_t* index, int64_t* value, int32_t clear);

/*
 * paged_kv_write -- store each new token's K and V rows into its slot of the paged pools
 * (the write step of a decode or prefill step: "vLLM-Style Llama Inference Engine",
 * How it works, step 3; the mini-vLLM README's per-sequence K/V write loop into the block
 * pool, done here as one scatter).
 *
 *   k, v           16-bit elements [num_tokens][num_kv_heads][head_dim]  (read); bf16 or
 *                  fp16 alike, the call moves bit patterns
 *   slot_mapping   int64 [num_tokens]; token t goes to slot s = slot_mapping[t], i.e. block
 *                  s / block_size, offset s % block_size. s < 0: token skipped (padding).
 *                  Non-negative slots must be distinct and < num_blocks*block_size; a slot
 *                  outside the pool is not written.
 *   k_cache, v_cache  [num_blocks][block_size][num_kv_heads][head_dim], same format as k/v, modified in
 *                  place; only the addressed rows change. Bits are copied unchanged (no
 *                  float conversion), so any payload, NaN included, is preserved.
 * Requirements: num_tokens >= 0 (0 = no-op), num_blocks >= 1, block_size >= 1,
 * num_kv_heads >= 1, head_dim >= 1, num_kv_heads*head_dim a multiple of 8.
 */
int paged_kv_write(const uint16_t* k, const uint16_t* v, const int64_t* slot_mapping,
                   int64_t num_tokens, uint16_t* k_cache, uint16_t* v_cache,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, hipStream_t stream);

/*
 * paged_kv_write_rope -- rotary position embedding at absolute positions fused with the KV
 * write: keys are rotated at their absolute positions before they enter the cache (llm-stack,
 * Serving engine / KV cache bullet), by a rotation of pairs of components with sine and cosine
 * ("tiny-vLLM" blog, CUDA Kernel Engineering: RoPE).
 *
 *   For token t at position positions[t] and pair i of every head vector:
 *     theta = fp32(positions[t]) * inv_freq[i]   (fp32 product)
 *     (x0, x1) -> (x0*cos(theta) - x1*sin(theta), x1*cos(theta) + x0*sin(theta))
 *   computed in fp32 and rounded to bf16 (nearest even). Pairs are (i, i + D/2) when
 *   interleaved == 0 (half split) or (2i, 2i+1) when interleaved == 1.
 *   q [T][Hq][D] -> q_out [T][Hq][D] (rotated; q_out may be q itself);
 *   k [T][Hkv][D] rotated and v [T][Hkv][D] copied to slot slot_mapping[t] of the pools, as
 *   paged_kv_write does (negative slot: nothing stored; q_out is still written).
 *   inv_freq       fp32 [D/2], the caller's per-pair frequencies (e.g. base^(-2i/D), with any
 *                  long-context rescaling already applied)
 * Requirements: head_dim a multiple of 8, at most 512; v and v_cache 16-byte aligned. Status
 * codes and asynchrony as above.
 */
int paged_kv_write_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* positions, const float* inv_freq, int32_t interleaved,
                        const int64_t* slot_mapping, int64_t num_tokens, uint16_t* q_out,
                        uint16_t* k_cache, uint16_t* v_cache, int64_t num_blocks,
                        int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, hipStream_t stream);

/*
 * paged_decode_workspace_bytes -- bytes of device workspace paged_decode_attention needs
 * for these sizes (0 when the call never splits a sequence and block_size is 16): the split
 * partials, then, for blocks larger than 16 tokens, the table of 16-token block ids.
 * `partition_tokens` has the same meaning as in paged_decode_attention; for 0 (automatic)
 * the bound covers every partition size the automatic choice can make.
 */
size_t paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t partition_tokens);

/*
 * paged_decode_attention -- one-token grouped-query decode attention over the paged cache
 * ("vLLM-Style Llama Inference Engine", How it works, step 4; mini-vLLM README, paged
 * KV-cache paragraph and its test of the paged kernel against dense attention on scattered
 * blocks; llm-stack, Serving engine / KV cache bullet: the decode query sees every cached
 * key, no causal mask).
 *
 *   out[b][h][:] = sum_t softmax_t(scale * q[b][h] . K_b[t][g]) V_b[t][g],  g = h / G,
 *   over t = 0 .. context_lens[b]-1, where K_b[t] / V_b[t] is the row at logical position t
 *   read through block_tables[b]. context_lens[b] == 0 gives out[b] = 0.
 *
 *   q              bf16 [batch][num_q_heads][head_dim]
 *   k_cache, v_cache  bf16 [num_blocks][block_size][num_kv_heads][head_dim]
 *   block_tables   int32 [batch][max_blocks_per_seq]; entries at j >= ceil(L_b/block_size)
 *                  are never read (may be -1)
 *   context_lens   int32 [batch], 0 <= L_b <= max_blocks_per_seq*block_size
 *   scale          applied in fp32 to the fp32 dot product (typically 1/sqrt(head_dim))
 *   out            fp32 [batch][num_q_heads][head_dim] (written)
 *   workspace      device scratch of >= paged_decode_workspace_bytes(...) bytes, 16-byte
 *                  aligned, or NULL/0 when that size is 0. Contents need no initialisation;
 *                  calls that may run concurrently must not share one workspace.
 *   partition_tokens  0: choose automatically from the sizes and the device; -1: never
 *                  split a sequence; > 0: split each sequence into partitions of this many
 *                  tokens (a multiple of block_size) whose partial softmax results are
 *                  merged by a log-sum-exp reduction.
 * Supported: head_dim in {64, 128}; block_size a multiple of 16 up to 1024 (other sizes:
 * PAGEDKV_ERR_UNSUPPORTED); num_q_heads / num_kv_heads in {1, 2, 3, 4, 8} (other ratios up
 * to 16 with the matrix-core kernel). The kernels read 16-token blocks: a pool of larger
 * blocks is read as the same memory cut into 16-token blocks, through a table of their ids
 * (batch x max_blocks_per_seq x block_size/16 int32) that one small extra launch writes into
 * the workspace, after the split partials. num_blocks * block_size / 16 must fit in int32.
 * Accuracy: scores, softmax statistics and sums in fp32; the attention weights enter the
 * matrix product with V as a bf16 hi + lo pair (about 16 significant bits). Measured
 * |out - exact| stays below 5e-5 on the test workloads (logits of std up to 3); the tests
 * bound it by 2e-3.
 */
int paged_decode_attention(const uint16_t* q, const uint16_t* k_cache,
                           const uint16_t* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, float* out, void* workspace, size_t workspace_bytes,
                           int32_t partition_tokens, hipStream_t stream);

/*
 * paged_decode_attention_typed -- paged_decode_attention in other formats:
 *   kv_dtype       format of q, k_cache and v_cache: PAGEDKV_DTYPE_BF16 or PAGEDKV_DTYPE_F16
 *   out            [batch][num_q_heads][head_dim] in out_dtype (written)
 *   out_dtype      PAGEDKV_DTYPE_F32, or kv_dtype (the fp32 result rounded to nearest even)
 * Other pairs return PAGEDKV_ERR_UNSUPPORTED. Everything else, the workspace included, is as
 * in paged_decode_attention (whose formats are bf16 in, fp32 out). Accumulation is fp32 in
 * every format. With fp16 inputs the attention weights enter the matrix product as an fp16
 * hi + lo pair scaled by 2^7 (the scale cancels in the normalisation), so weights down to
 * 2^-31 of the largest still count; a 16-bit output adds its own rounding, at most half a
 * unit in its last place.
 */
int paged_decode_attention_typed(const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t partition_tokens, hipStream_t stream);

/* Kernel families for paged_decode_attention_ex. */
typedef enum {
  PAGEDKV_KERNEL_AUTO = 0,  /* the library's choice for the shape (the default path): for
                               contexts over 1024 tokens MFMA_HEADWAVE, or MFMA_STREAM when
                               batch * num_kv_heads exceeds a quarter of the compute units and
                               the head-per-wave plan would have more workgroups than compute
                               units; for shorter contexts MFMA */
  PAGEDKV_KERNEL_VALU = 1,  /* fp32 vector-ALU dot products and accumulation; a workgroup's
                               4 waves split one (sequence, KV head) partition */
  PAGEDKV_KERNEL_MFMA = 2,  /* bf16 matrix-core (MFMA) tiles, fp32 accumulation; a
                               workgroup's 4 waves split one (sequence, KV head) partition */
  PAGEDKV_KERNEL_MFMA_HEADWAVE = 3, /* MFMA tiles; a workgroup's 4 waves take 4 KV heads of
                               one (sequence, partition), one wave per head */
  PAGEDKV_KERNEL_MFMA_STREAM = 4  /* MFMA tiles, one wave per KV head as in MFMA_HEADWAVE; a
                               persistent grid (one workgroup per compute unit) counts the
                               batch's work on the device from context_lens and gives every
                               workgroup an equal contiguous slice of it (32-token pairs of
                               (sequence, 4 KV heads)), so ragged batches stay balanced; a
                               slice that spans sequences leaves one partial per sequence for
                               the partition merge. Contexts over 1024 tokens only. It always
                               splits: partition_tokens 0 lets the library bound the partials
                               (at most 16 per sequence), > 0 sets the least tokens per
                               workgroup, -1 returns PAGEDKV_ERR_UNSUPPORTED */
} pagedkv_kernel;

/*
 * paged_decode_attention_ex -- paged_decode_attention_typed with two extra controls, for
 * comparison and profiling:
 *   kernel         a pagedkv_kernel value (PAGEDKV_ERR_UNSUPPORTED if that family has no
 *                  build for the shape);
 *   ev_begin, ev_end  if non-NULL, recorded on `stream` immediately before and after the
 *                  main attention kernel (not the partition merge), so the caller can time
 *                  that kernel alone with hipEventElapsedTime.
 */
int paged_decode_attention_ex(const uint16_t* q, const uint16_t* k_cache,
                              const uint16_t* v_cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                              void* workspace, size_t workspace_bytes,
                              int32_t partition_tokens, int32_t kernel, hipEvent_t ev_begin,
                              hipEvent_t ev_end, hipStream_t stream);

/*
 * paged_decode_step -- the whole decode step in one call: the KV write of paged_kv_write for
 * one new token per sequence, then paged_decode_attention_ex over the updated pools ("vLLM-Style
 * Llama Inference Engine with Tensor Parallelism", How it works, steps 3-4: each rank writes
 * its paged KV cache, then one-token decode attends over it).
 *
 *   k_new, v_new   [batch][num_kv_heads][head_dim], kv_dtype: sequence b's new K and V rows
 *   slot_mapping   int64 [batch]: slot for row b (< 0 or outside the pool: not stored)
 *   k_cache, v_cache  as in paged_decode_attention, modified in place at those slots
 *   everything else as in paged_decode_attention_ex (kernel, events around the main kernel)
 *
 * The result equals paged_kv_write(k_new, v_new, slot_mapping, batch, ...) followed by
 * paged_decode_attention_ex(...) on the same stream, provided the decode-step layout holds:
 * slot_mapping[b] is the slot that block_tables[b] gives for position context_lens[b] - 1
 * (the new token is the last position), or negative. The matrix-core kernels then store the
 * rows and read that position from k_new / v_new within one launch, with no separate write
 * launch; a slot that addresses some other position this call reads gives an undefined
 * result. The vector-ALU family (kernel = PAGEDKV_KERNEL_VALU) issues the write as its own
 * launch before the attention.
 */
int paged_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, float scale, int32_t kv_dtype, void* out,
                      int32_t out_dtype, void* workspace, size_t workspace_bytes,
                      int32_t partition_tokens, int32_t kernel, hipEvent_t ev_begin,
                      hipEvent_t ev_end, hipStream_t stream);

/* Size of the device scratch array paged_decode_step_noalloc uses (per device). */
#define PAGEDKV_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * paged_decode_step_noalloc -- paged_decode_step for callers that cannot allocate device
 * memory: code recorded under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. It takes no workspace. The split partials and, for blocks larger than 16 tokens,
 * the table of 16-token block ids live in a file-scope device array of
 * PAGEDKV_STATIC_SCRATCH_BYTES bytes inside the library, one per device, held until the
 * process ends; the call allocates and frees nothing (no hipMalloc / hipFree, no allocating
 * library routine).
 *
 *   Arguments as in paged_decode_step, without workspace and workspace_bytes. The result
 *   equals paged_decode_step with a workspace of its own.
 *   Scratch bound: a call whose plan needs more than PAGEDKV_STATIC_SCRATCH_BYTES (for 16-token
 *   blocks: batch * num_q_heads * partitions * (head_dim + 2) * 4 bytes when it splits, 0 when
 *   it does not; paged_decode_plan gives the partition count) returns PAGEDKV_ERR_WORKSPACE
 *   before anything is enqueued, with the sizes in paged_kv_last_error().
 *   Sharing: every call on one device uses that device's one array, which keeps the last
 *   call's contents; no part of it needs to start at zero (every value a call reads was
 *   written by the same call). Calls that may overlap on one device (other streams, other
 *   threads) race on the array and must be serialised by the caller.
 *   Set-up: the first call on a device looks up the array's device address (with that device
 *   current) and keeps it; a failure there returns PAGEDKV_ERR_HIP.
 */
int paged_decode_step_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, float scale, int32_t kv_dtype, void* out,
                              int32_t out_dtype, int32_t partition_tokens, int32_t kernel,
                              hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream);

/*
 * paged_decode_step_rope -- paged_decode_step with the rotary embedding of paged_kv_write_rope
 * in front: q and k_new are rotated at positions[b] before they are used ("tiny-vLLM" blog,
 * CUDA Kernel Engineering: RoPE; llm-stack, Serving engine / KV cache bullet: keys enter the
 * cache rotated at their absolute positions).
 *
 *   q              [batch][num_q_heads][head_dim] bf16, not rotated; left unchanged
 *   k_new, v_new   as in paged_decode_step (k_new not rotated)
 *   positions      int32 [batch]: the absolute position of sequence b's new token
 *   inv_freq, interleaved  as in paged_kv_write_rope (inv_freq 16-byte aligned)
 *   q_out          [batch][num_q_heads][head_dim] bf16: receives the rotated q; must not
 *                  overlap q (the attention reads q while q_out is written)
 *   everything else as in paged_decode_step
 *
 * The result (q_out, the pools, out) equals, bit for bit, paged_kv_write_rope(q, k_new, v_new,
 * positions, inv_freq, interleaved, slot_mapping, batch, q_out, ...) followed by
 * paged_decode_attention_ex(q_out, ...), under the decode-step layout of paged_decode_step.
 * The matrix-core kernels do all of it in one launch: the rotation happens in registers on the
 * pieces of q and of the new key each lane already holds for its matrix tiles. The vector-ALU
 * family issues paged_kv_write_rope as its own launch. bf16 inputs only
 * (PAGEDKV_ERR_UNSUPPORTED otherwise); head_dim 64 or 128 as for the attention.
 */
int paged_decode_step_rope(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* positions, const float* inv_freq, int32_t interleaved,
                           const int64_t* slot_mapping, uint16_t* q_out, uint16_t* k_cache,
                           uint16_t* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                           void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                           int32_t kernel, hipEvent_t ev_begin, hipEvent_t ev_end,
                           hipStream_t stream);

/*
 * paged_decode_plan -- the launch paged_decode_attention_ex would make for these sizes on
 * the current device, without launching: number of sequence partitions, tokens per
 * partition, and the kernel family (a pagedkv_kernel value, never AUTO). For the stream
 * family: partial slots per (sequence, KV head) and the least tokens per workgroup. partition_tokens
 * and kernel as in paged_decode_attention_ex. Returns a status; the outputs are written on
 * PAGEDKV_OK (chosen_kernel may be NULL). The plan depends on the device only through its
 * compute-unit count; if the environment variable PAGEDKV_CU_COUNT holds a positive integer,
 * every call of the library uses that count instead (meant for planning without a device).
 */
int paged_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                      int32_t partition_tokens, int32_t kernel, int32_t* num_partitions,
                      int32_t* tokens_per_partition, int32_t* chosen_kernel);

/*
 * paged_prefill_attention -- multi-query causal attention over the paged cache: prefill,
 * chunked prefill and recompute (the Llama engine's causal prefill / recomputation,
 * "vLLM-Style Llama Inference Engine with Tensor Parallelism", Features and scope /
 * Implemented; the ragged attention without padding, gathering by block table, planned in
 * llm-stack's Roadmap).
 *
 *   Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Q_b rows), which are
 *   its last Q_b logical positions: row i sits at position p = context_lens[b] - Q_b + i and
 *   out[row][h][:] = sum_{t<=p} softmax_t(scale * q[row][h] . K_b[t][g]) V_b[t][g], g = h/G.
 *   The rows' own keys must already be in the cache (write them with paged_kv_write first).
 *
 *   q              bf16 [num_tokens][num_q_heads][head_dim], the sequences' rows back to back
 *   cu_seqlens_q   int32 [batch+1], 0 = cu[0] <= cu[1] <= ... <= cu[batch] = num_tokens
 *   max_q_len      >= max_b Q_b (sizes the grid on the host without reading cu_seqlens_q)
 *   k_cache, v_cache, block_tables, context_lens, scale: as in paged_decode_attention;
 *                  Q_b <= context_lens[b] (rows whose position would be negative get 0)
 *   out            fp32 [num_tokens][num_q_heads][head_dim] (written)
 * Supported: head_dim in {64, 128}; block_size 16, 32, 64, ... 1024 (blocks larger than 16
 * tokens are read as the same memory cut into 16-token blocks; num_blocks * block_size / 16
 * must fit in int32); num_q_heads / num_kv_heads in 1..16.
 * Needs no workspace. Asynchronous on `stream`; status codes as above.
 */
int paged_prefill_attention(const uint16_t* q, const int32_t* cu_seqlens_q, int64_t num_tokens,
                            int32_t max_q_len, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, float scale, float* out, hipStream_t stream);

/*
 * paged_prefill_attention_ex -- paged_prefill_attention in other formats and with the work
 * split chosen by the caller:
 *   kv_dtype, out_dtype  formats of q and the caches, and of out, as in
 *                  paged_decode_attention_typed (paged_prefill_attention is bf16 in, fp32 out)
 *   row_blocks     number of 16-row blocks of queries each wave carries through one pass
 *                  over the keys (1, 2 or 4), or 0 to let the library choose from the sizes
 *                  and the device (what paged_prefill_attention does). Results agree across
 *                  choices up to fp32 rounding of the same sums. Any other value returns
 *                  PAGEDKV_ERR_SHAPE.
 */
int paged_prefill_attention_ex(const uint16_t* q, const int32_t* cu_seqlens_q,
                               int64_t num_tokens, int32_t max_q_len, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                               int32_t row_blocks, hipStream_t stream);

/*
 * paged_prefill_attention_split -- paged_prefill_attention_ex with the keys of each query
 * tile optionally cut into partitions, each computed by workgroups of its own and combined by
 * the log-sum-exp merge of the decode path (the running-max rescaling of the tiled online
 * softmax, llm-stack, Attention kernel section, applied across partitions; the split-K kernel
 * the "vLLM-Style Llama Inference Engine with Tensor Parallelism" page lists as out of its
 * scope). It shortens the serial chain of keys when a batch has few query rows against long
 * contexts, such as a short chunk appended to a long cached prefix.
 *
 *   workspace, workspace_bytes  device memory of at least paged_prefill_workspace_bytes(...)
 *                  bytes, 16-byte aligned, used only while the call's kernels run; NULL / 0 is
 *                  allowed when the plan does not split. Contents need no initialisation.
 *                  Calls that may overlap (other streams) need their own workspace.
 *   partition_tokens  keys per partition: 0 lets the library choose (it splits only when the
 *                  query tiles cannot fill the device and contexts may exceed 2048 keys, into
 *                  at most 3 partitions of at least 512 keys), -1 never splits, > 0 forces
 *                  that size, which must be a multiple of 32 (else PAGEDKV_ERR_SHAPE).
 *   Other arguments as in paged_prefill_attention_ex. A split adds a second launch (the
 *   merge) on `stream`. Results agree with the unsplit call up to fp32 rounding of the same
 *   sums; a row that sees a single key still returns that value row exactly.
 */
int paged_prefill_attention_split(const uint16_t* q, const int32_t* cu_seqlens_q,
                                  int64_t num_tokens, int32_t max_q_len,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, float scale,
                                  int32_t kv_dtype, void* out, int32_t out_dtype,
                                  int32_t row_blocks, void* workspace, size_t workspace_bytes,
                                  int32_t partition_tokens, hipStream_t stream);

/*
 * paged_prefill_workspace_bytes -- bytes of workspace paged_prefill_attention_split needs
 * (0 when it never splits for these sizes). For partition_tokens 0 the bound covers every
 * plan the automatic choice can make; it does not depend on the device.
 */
size_t paged_prefill_workspace_bytes(int64_t num_tokens, int32_t num_q_heads, int32_t head_dim,
                                     int32_t max_blocks_per_seq, int32_t block_size,
                                     int32_t partition_tokens);

/*
 * paged_prefill_plan -- the launch paged_prefill_attention_split would make for these sizes
 * on the current device, without launching: 16-row blocks per wave, key partitions per query
 * tile (1: no split) and keys per partition. Arguments as in paged_prefill_attention_split;
 * outputs are written on PAGEDKV_OK. PAGEDKV_CU_COUNT overrides the compute-unit count as in
 * paged_decode_plan (the choice of row_blocks = 0 also asks the runtime for the kernels'
 * occupancy, which needs a device).
 */
int paged_prefill_plan(int64_t num_tokens, int32_t max_q_len, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t row_blocks,
                       int32_t partition_tokens, int32_t* row_blocks_used,
                       int32_t* num_partitions, int32_t* keys_per_partition);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
