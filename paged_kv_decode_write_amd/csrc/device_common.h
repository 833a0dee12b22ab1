// Device-side helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pagedkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Element formats (the values of the C ABI's pagedkv_dtype).
enum : int { kDtBf16 = 0, kDtF16 = 1, kDtF32 = 2 };

// 16-bit input element -> fp32, exact for both formats: a bf16 value is the upper half of an
// fp32 bit pattern; an fp16 value converts with v_cvt_f32_f16.
template <int KT> __device__ __forceinline__ float in_lo(uint32_t w) {
  if constexpr (KT == kDtF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  else return __uint_as_float(w << 16);
}
template <int KT> __device__ __forceinline__ float in_hi(uint32_t w) {
  if constexpr (KT == kDtF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return __uint_as_float(w & 0xffff0000u);
}

template <int KT> __device__ __forceinline__ void unpack8(const uint4& w, float (&f)[8]) {
  f[0] = in_lo<KT>(w.x); f[1] = in_hi<KT>(w.x);
  f[2] = in_lo<KT>(w.y); f[3] = in_hi<KT>(w.y);
  f[4] = in_lo<KT>(w.z); f[5] = in_hi<KT>(w.z);
  f[6] = in_lo<KT>(w.w); f[7] = in_hi<KT>(w.w);
}

// Makes an fp32 value opaque to the optimiser, so the operation that produced it is rounded
// to fp32 first. Without it, a product feeding an fp16 conversion may be contracted into one
// v_fma_mix*_f16 (a single rounding of the exact product): close, but not the fp32 result
// rounded, which is what a 16-bit output is defined to hold. Not volatile: a volatile asm
// counts as a possible memory write, and one ahead of a loop would stop the compiler from
// reading the block table through the scalar cache inside it.
__device__ __forceinline__ float materialize_f32(float f) {
  asm("" : "+v"(f));
  return f;
}

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)materialize_f32(f));
}
// fp32 -> fp16 with v_cvt_f16_f32 (round to nearest even; overflow gives infinity).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)materialize_f32(f));
}

// Rotary embedding of one pair (x0, x1) by an angle with cosine c and sine s, written with
// explicit fused multiply-adds so every kernel that rotates produces the same bits:
// y0 = x0 c - x1 s, y1 = x1 c + x0 s, each the fma of one product with the other one rounded.
__device__ __forceinline__ void rope_rotate(float x0, float x1, float c, float s, float& y0,
                                            float& y1) {
  y0 = __builtin_fmaf(x0, c, -(x1 * s));
  y1 = __builtin_fmaf(x1, c, x0 * s);
}

// Output stores: one value, or four consecutive values (index a multiple of 4), in the
// output format OT.
template <int OT> __device__ __forceinline__ void store_out(void* out, size_t i, float v) {
  if constexpr (OT == kDtF32) static_cast<float*>(out)[i] = v;
  else if constexpr (OT == kDtBf16) static_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(v);
  else static_cast<uint16_t*>(out)[i] = f32_to_f16_rne(v);
}
template <int OT>
__device__ __forceinline__ void store_out4(void* out, size_t i, float a, float b, float c,
                                           float d) {
  if constexpr (OT == kDtF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = make_float4(a, b, c, d);
  } else {
    uint16_t h[4];
    if constexpr (OT == kDtBf16) {
      h[0] = f32_to_bf16_rne(a); h[1] = f32_to_bf16_rne(b);
      h[2] = f32_to_bf16_rne(c); h[3] = f32_to_bf16_rne(d);
    } else {
      h[0] = f32_to_f16_rne(a); h[1] = f32_to_f16_rne(b);
      h[2] = f32_to_f16_rne(c); h[3] = f32_to_f16_rne(d);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i) =
        make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  }
}

// v_exp_f32: 2^x, with 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a row of 16 lanes (gfx9 DPP controls).
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor3 = 0x1B,      // quad_perm [3,2,1,0]
  kDppRowMirror = 0x140,    // lane i <- lane 15-i within the row
  kDppRowHalfMirror = 0x141 // lane i <- lane 7-i within each half row
};

template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, true));
}

// Sum over groups of N consecutive lanes (N in {8, 16}); every lane of a group receives the
// group sum, bit-identical across the group (each butterfly pairs equal operands).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group size");
  if constexpr (N == 16) v += dpp<kDppRowMirror>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppQuadXor3>(v);
  v += dpp<kDppQuadXor1>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Max / sum over lanes l, l^16, l^32, l^48 (the four lanes of a 16-lane column), every lane
// receiving the result, with gfx950's v_permlane32_swap / v_permlane16_swap (no LDS path, no
// address arithmetic). Called with both operands equal, a swap leaves lane l holding its own
// value in one result and its partner's in the other, whichever half moves where, so the
// symmetric max / sum of the two is the pairwise reduction.
__device__ __forceinline__ float row4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Partition index of a decode work unit. Units are numbered row-major with the partition
// fastest (row = unit / nparts), and the hardware deals workgroups to the 8 XCDs round-robin by
// block index, so with nparts sharing a factor with 8 the partition index would be tied to the
// XCD (with nparts = 8, partition p of every row on XCD p). In a ragged batch early partitions
// carry far more work than late ones, which are empty for short contexts, and the XCDs that
// drew the early ones would bound the time. Rotating each row's partitions by row / m, with
// m = 8 / gcd(nparts, 8), lands every partition index on each XCD equally often across rows.
// A permutation of the partitions within each row.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_balanced_part(int unit, int nparts) {
  const int row = unit / nparts;
  const int slot = unit - row * nparts;
  const int low = nparts & -nparts;  // the largest power of two dividing nparts
  const int m = kXcds / (low < kXcds ? low : kXcds);
  return (slot + row / m) % nparts;
}

// A partition that starts past its sequence's context (only in a split launch: partition 0
// never exits early) marks its G query rows as holding no keys, max -inf and sum 0, which is
// all the merge reads of it. Thread i < G of the exiting unit marks row i of KV head g.
// neg_inf is -inf (a kernel may pass it through an empty asm first, see keep_issued).
__device__ __forceinline__ void mark_empty_partition(const DecodeArgs& a, int b, int g,
                                                     int part, int i,
                                                     float neg_inf = kNegInf) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (i >= G) return;
  const size_t pr = ((size_t)b * a.num_q_heads + (size_t)g * G + i) * a.nparts + part;
  a.ws_ml[pr * 2 + 0] = neg_inf;
  a.ws_ml[pr * 2 + 1] = 0.f;
}

}  // namespace pagedkv
