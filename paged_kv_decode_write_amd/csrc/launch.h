// Internal interface between the C-ABI host layer (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace pagedkv {

// Arguments of one decode-attention launch, already validated by the host layer.
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;        // [B][Hq][D] in the output format
  float* ws_acc;    // [B][Hq][nparts][D] unnormalised partial outputs (split only)
  float* ws_ml;     // [B][Hq][nparts][2] partial (max, sum) in log2 units (split only)
  int32_t max_blocks;  // MB, block-table row length
  int32_t batch, num_q_heads, num_kv_heads, head_dim, block_size;
  int64_t num_blocks;
  float scale_log2;     // scale * log2(e)
  int32_t nparts;       // partitions per sequence (1 = write out directly)
  int32_t part_tokens;  // tokens per partition, a multiple of block_size
  int32_t kv_dtype;     // format of q and the caches: kDtBf16 or kDtF16
  int32_t out_dtype;    // kDtF32 or kv_dtype
  // Fused decode step (k_new != nullptr): sequence b's new K / V rows k_new[b], v_new[b]
  // ([B][Hkv][D]) are stored at slot_mapping[b] of the writable pools and used for position
  // context_lens[b] - 1 when that slot is the one the block table gives for it.
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* slot_mapping;
  uint16_t* k_cache_w;
  uint16_t* v_cache_w;
  // Fused decode step with rotary embedding (positions != nullptr): q and the new keys are
  // rotated at positions[b] with inv_freq ([D/2], half or interleaved pairing) before use; the
  // rotated q goes to q_out, the rotated key to the cache.
  const int32_t* positions;
  const float* inv_freq;
  int32_t interleaved;
  uint16_t* q_out;
  // Evenly divided (stream-K) launch: a workgroup takes at least this many 32-token pairs of
  // the batch's work; nparts is then the number of partial slots per (sequence, KV head).
  int32_t sk_min_pairs;
  // Nonzero: the slices are weighted by the XCD each workgroup runs on (the device whole).
  int32_t sk_xcd_weights;
};

// Arguments of one multi-query causal (prefill) launch, already validated.
struct PrefillArgs {
  const uint16_t* q;             // [T][Hq][D]
  const int32_t* cu_seqlens_q;   // [B+1]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;                     // [T][Hq][D] in the output format
  int32_t max_blocks;
  int32_t batch, num_q_heads, num_kv_heads, head_dim, block_size;
  int64_t num_blocks;
  float scale_log2;
  int32_t ntiles;  // query tiles per sequence (ceil(max_q_len / tokens per workgroup))
  int32_t nb;      // 16-row N blocks per wave: 1, 2 or 4
  int32_t kv_dtype, out_dtype;  // as in DecodeArgs
  // Key split: each query tile's keys are cut into partitions of part_keys (a multiple of 32)
  // and each (tile, partition) is one workgroup, which leaves per-row partials for the
  // partition merge (the layout of DecodeArgs with the query tokens as the batch).
  int32_t nparts;     // partitions per query tile (1 = write out directly)
  int32_t part_keys;  // keys per partition
  float* ws_acc;      // [T][Hq][nparts][D] (split only)
  float* ws_ml;       // [T][Hq][nparts][2] (split only)
};

// Arguments of one rotary-embedding + KV-write launch, already validated.
struct RopeArgs {
  const uint16_t* q;        // [T][Hq][D]
  const uint16_t* k;        // [T][Hkv][D]
  const uint16_t* v;        // [T][Hkv][D]
  const int32_t* positions; // [T]
  const float* inv_freq;    // [D/2]
  const int64_t* slot_mapping;
  uint16_t* q_out;          // [T][Hq][D] (may alias q)
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t num_tokens, num_slots;
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t interleaved;
};

// Calls f(integral_constant<KT>, integral_constant<OT>) for the compiled (input, output)
// format pairs: bf16 or fp16 inputs, fp32 output or the input's own format.
template <class F>
hipError_t with_formats(int kv_dtype, int out_dtype, F&& f) {
  using B16 = std::integral_constant<int, 0>;
  using F16 = std::integral_constant<int, 1>;
  using F32 = std::integral_constant<int, 2>;
  if (kv_dtype == 0 && out_dtype == 2) return f(B16{}, F32{});
  if (kv_dtype == 0 && out_dtype == 0) return f(B16{}, B16{});
  if (kv_dtype == 1 && out_dtype == 2) return f(F16{}, F32{});
  if (kv_dtype == 1 && out_dtype == 1) return f(F16{}, F16{});
  return hipErrorInvalidValue;
}

// Each launcher returns hipSuccess or the launch error. `supported_*` report whether a
// compiled instance exists for the shape.
bool supported_valu(int head_dim, int group, int block_size);
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream);

bool supported_mfma(int head_dim, int group, int block_size);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// One wave per KV head, kHeadsPerGroup heads of a (sequence, partition) per workgroup.
hipError_t launch_decode_mfma_hw(const DecodeArgs& a, hipStream_t stream);
// The batch's work counted on the device and cut into equal slices, one per workgroup of
// `workgroups` (kHeadsPerGroup KV heads, one wave each); leaves partials for the merge.
hipError_t launch_decode_mfma_sk(const DecodeArgs& a, int workgroups, hipStream_t stream);

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream);
// The merge of the multi-query key split: rows are (token, query head); rows marked done are
// skipped and empty partitions' outputs are not read.
hipError_t launch_prefill_merge(const DecodeArgs& a, hipStream_t stream);

bool supported_prefill(int head_dim, int group, int block_size);
int prefill_rows_per_wave(int64_t num_tokens, int num_kv_heads, int head_dim, int group, int cus);
int prefill_tokens_per_group(int group, int nb);  // query tokens one workgroup covers
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_kv_write_rope(const RopeArgs& a, hipStream_t stream);

// Writes the 16-token-block view of a table of blocks of 16 * sub tokens: out is
// [batch][max_blocks * sub]; ids outside [0, num_blocks) become -1.
hipError_t launch_expand_table(const int32_t* table, int32_t batch, int32_t max_blocks,
                               int32_t sub, int64_t num_blocks, int32_t* out,
                               hipStream_t stream);

hipError_t launch_kv_write(const uint16_t* k, const uint16_t* v, const int64_t* slots,
                           int64_t num_tokens, uint16_t* k_cache, uint16_t* v_cache,
                           int64_t num_slots, int32_t row_elems, hipStream_t stream);

// Device-side validation (launched by the checked build before a call's kernels): codes of
// the first violation recorded, as paged_kv_check_status reports them.
constexpr int kCheckSlot = 1;    // slot id at or past the end of the pool
constexpr int kCheckLength = 2;  // context length negative or past the table width
constexpr int kCheckBlock = 3;   // a block id the context covers lies outside the pool
constexpr int kCheckQuery = 4;   // a query span that is negative, past num_tokens, longer
                                 // than its context or than max_q_len
hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t num_slots,
                              hipStream_t stream);
hipError_t launch_check_tables(const int32_t* tables, const int32_t* lens, int32_t batch,
                               int32_t max_blocks, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream);
hipError_t launch_check_queries(const int32_t* cu, const int32_t* lens, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int64_t num_tokens,
                                int32_t max_q_len, hipStream_t stream);
// Synchronises the current device, then reads (and with `clear` zeroes) its record:
// {code, index, value}.
hipError_t read_check_record(long long rec[3], bool clear);

// Waves per workgroup of the decode kernels; partitions are multiples of
// kWavesPerGroup * block_size tokens when split automatically.
constexpr int kWavesPerGroup = 4;
// KV heads (one wave each) per workgroup of the head-per-wave MFMA kernel.
#ifndef PAGEDKV_HEADS_PER_GROUP
#define PAGEDKV_HEADS_PER_GROUP 4
#endif
constexpr int kHeadsPerGroup = PAGEDKV_HEADS_PER_GROUP;

// log2(e), to turn natural-log scores into log2 units for v_exp_f32.
constexpr float kLog2eHost = 1.4426950408889634f;

}  // namespace pagedkv
