// Pieces of the fused decode step shared by the matrix-core decode kernels: which position
// takes the step's new K / V row, where the new-row loads read, and the stores of the new rows
// and of the rotated q ("vLLM-Style Llama Inference Engine with Tensor Parallelism", How it
// works, steps 3-4: each rank writes its paged KV cache, then one-token decode attends over it).
#pragma once

#include "launch.h"
#include "mfma_tiles.h"

namespace pagedkv {

// Fused decode step (a.k_new set): the position whose K / V come from the step's new rows
// instead of the cache, or -1. That is position L - 1 when the slot the step writes for
// sequence b is the one its block table gives for that position (the decode-step layout);
// otherwise the cache is read as it stands.
// sub_pos_of takes the values already read (slot = slots[b], entry = table[(L - 1) / 16]);
// step_sub_pos reads them. `slots` is the step's slot mapping (a.slot_mapping, or the same
// array through a pointer the caller knows no store reaches, so the read stays a scalar load).
__device__ __forceinline__ int sub_pos_of(const DecodeArgs& a, int64_t slot, int32_t entry,
                                          int L) {
  if (!a.k_new || L <= 0) return -1;
  const int64_t want = (int64_t)entry * 16 + (L - 1) % 16;
  return slot >= 0 && slot == want && slot < a.num_blocks * 16 ? L - 1 : -1;
}
__device__ __forceinline__ int step_sub_pos(const DecodeArgs& a, const int64_t* slots,
                                            const int32_t* table, int b, int L) {
  if (!a.k_new || L <= 0) return -1;
  return sub_pos_of(a, slots[b], table[(L - 1) / 16], L);
}
// The new token's slot, read once by a kernel that both tests it and stores there (-1
// without new rows), and the test on it.
__device__ __forceinline__ int64_t step_slot(const DecodeArgs& a, int b) {
  return a.k_new ? a.slot_mapping[b] : -1;
}
__device__ __forceinline__ int step_sub_pos_at(const DecodeArgs& a, int64_t slot,
                                               const int32_t* table, int L) {
  if (!a.k_new || L <= 0) return -1;
  return sub_pos_of(a, slot, table[(L - 1) / 16], L);
}

// Rows the fused step's new-row loads read for KV head g of sequence b: the step's new K / V
// rows when the call has them; otherwise slot 0 of head g in the pools, which exists for any
// batch (the pool holds at least one block) and whose values are then never used.
__device__ __forceinline__ const uint16_t* new_k_row(const DecodeArgs& a, int b, int g, int D) {
  return a.k_new ? a.k_new + ((size_t)b * a.num_kv_heads + g) * D : a.k_cache + (size_t)g * D;
}
__device__ __forceinline__ const uint16_t* new_v_row(const DecodeArgs& a, int b, int g, int D) {
  return a.v_new ? a.v_new + ((size_t)b * a.num_kv_heads + g) * D : a.v_cache + (size_t)g * D;
}

// Fused decode step: store KV head g's slice of sequence b's new K and V rows at
// slot_mapping[b] (negative or outside the pool: nothing), 16 bytes per lane, K from lanes
// 0..D/8-1 and V from lanes 32..32+D/8-1 of one wave. Only the launch unit that reads
// position L - 1 (or partition 0 when L = 0) calls it, so every slice is written once and no
// unit of the launch reads it back (the owner takes that position from the new rows).
template <int D>
__device__ __forceinline__ void step_store(const DecodeArgs& a, const int64_t* slots, int b,
                                           int g, int lane) {
  const int64_t slot = slots[b];
  if (slot < 0 || slot >= a.num_blocks * 16) return;
  const size_t src = ((size_t)b * a.num_kv_heads + g) * D;
  const size_t dst = ((size_t)slot * a.num_kv_heads + g) * D;
  const int i = lane & 31;
  if (i < D / 8) {
    const uint4* from = reinterpret_cast<const uint4*>((lane < 32 ? a.k_new : a.v_new) + src);
    uint4* to = reinterpret_cast<uint4*>((lane < 32 ? a.k_cache_w : a.v_cache_w) + dst);
    to[i] = from[i];
  }
}

// The same store from a wave's registers (the new rows as loaded, or the rotated key row of a
// RoPE step), at a slot already read: the lanes with n16 == 0 hold the whole K row (chunks
// 32ch + 8kg), the lanes with kg == 0 the whole V row (EPL columns at EPL * n16).
template <int D, int NCH, int EPL>
__device__ __forceinline__ void step_store_regs_at(const DecodeArgs& a, int64_t slot, int g,
                                                   const NewRow<NCH, EPL>& r, int n16, int kg) {
  if (slot < 0 || slot >= a.num_blocks * 16) return;
  const size_t dst = ((size_t)slot * a.num_kv_heads + g) * D;
  if (n16 == 0) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      *reinterpret_cast<uint4*>(a.k_cache_w + dst + 32 * ch + 8 * kg) = r.k[ch];
  }
  if (kg == 0) r.v.store(a.v_cache_w + dst + EPL * n16);
}
template <int D, int NCH, int EPL>
__device__ __forceinline__ void step_store_regs(const DecodeArgs& a, const int64_t* slots,
                                                int b, int g, const NewRow<NCH, EPL>& r,
                                                int n16, int kg) {
  step_store_regs_at<D>(a, slots[b], g, r, n16, kg);
}

// RoPE step, part 2 (part 1 is rope_pieces on the loaded q and new-key pieces): the rotated q
// rows of this wave's heads, from registers. Issued after the block loop, as the step store
// is, so that no store precedes the loop's block-table reads.
template <int D, int NCH>
__device__ __forceinline__ void store_q_out(const DecodeArgs& a, const uint4 (&qb)[NCH], int b,
                                            int g, int G, int n16, int kg) {
  if (n16 >= G) return;
  uint16_t* o = a.q_out + ((size_t)b * a.num_q_heads + (size_t)g * G + n16) * D + 8 * kg;
#pragma unroll
  for (int c = 0; c < NCH; ++c) *reinterpret_cast<uint4*>(o + 32 * c) = qb[c];
}

}  // namespace pagedkv
