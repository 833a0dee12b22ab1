// Device-side helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pagedkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// bf16 -> fp32 is exact: a bf16 value is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
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

}  // namespace pagedkv
