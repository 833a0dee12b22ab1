// Paged one-token decode attention, vector-ALU kernel (fp32 dot products and accumulate; bf16
// or fp16 inputs, output in fp32 or in the input format).
//
// Computes, for every sequence b and query head h, softmax(scale * q[b,h] . K^T) V over the
// context_lens[b] positions read through block_tables[b] (mini-vLLM README, paged KV-cache
// paragraph; "vLLM-Style Llama Inference Engine with Tensor Parallelism", How it works,
// step 4), with grouped-query heads (same page, Implemented) and a tiled online softmax with
// fp32 accumulation (llm-stack, Attention kernel section).
//
// Work decomposition (one workgroup = 4 waves):
//   workgroup <- (sequence b, KV head g, partition p of the sequence's tokens).
//   All G = Hq/Hkv query heads that share KV head g are packed into the workgroup, so every
//   K/V byte fetched from HBM serves G heads.
//   Wave w of the workgroup takes the partition's blocks w, w+4, w+8, ...
// Lane layout inside a wave, for one block of 16 tokens of head g (each token row is D bf16
// = D*2 contiguous bytes, rows Hkv*D*2 bytes apart):
//   LPR = D/8 lanes cover one row with 16-byte loads; RPL = 64/LPR rows per wave load;
//   lane = r0*LPR + col holds columns col*8..col*8+7 of rows r0, r0+RPL, r0+2*RPL, ...
//   q . k partial sums are reduced across the LPR lanes of a row with DPP; after that every
//   lane of the row holds the full scores of its rows, and the same lanes accumulate p*V for
//   the same rows and their own columns, so no score ever has to be broadcast.
//   Each row group r0 keeps its own running max / sum / accumulator; row groups and waves
//   are merged once at the end with the log-sum-exp rule.
// Scores are kept in log2 units (scale * log2 e folded in) and exponentiated with v_exp_f32.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

template <int D, int G, int BS, int NW, int KT, int OT>
__global__ void __launch_bounds__(NW * 64)
decode_valu_kernel(const DecodeArgs a) {
  constexpr int LPR = D / 8;        // lanes per token row
  constexpr int RPL = 64 / LPR;     // rows per wave-wide load
  constexpr int NI = BS / RPL;      // loads per block
  static_assert(BS % RPL == 0, "block size must be a multiple of rows per load");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane % LPR;
  const int r0 = lane / LPR;

  const int nparts = a.nparts;
  const int Hkv = a.num_kv_heads;
  const int unit = blockIdx.x;
  const int part = xcd_balanced_part(unit, nparts);
  const int g = (unit / nparts) % Hkv;
  const int b = unit / (nparts * Hkv);
  const int Hq = a.num_q_heads;

  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int tok0 = part * a.part_tokens;
  if (tok0 >= L && !(L == 0 && part == 0)) {  // partition past the end: nothing to do
    if (wave == 0) mark_empty_partition(a, b, g, part, lane);
    return;
  }
  const int tok1 = min(tok0 + a.part_tokens, L);
  const int blk0 = tok0 / BS;
  const int blk1 = (tok1 + BS - 1) / BS;

  // q rows of the G heads, this lane's 8 columns, as fp32.
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        a.q + ((size_t)b * Hq + (size_t)g * G + h) * D + col * 8);
    unpack8<KT>(w, qf[h]);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  }

  const size_t row_stride = (size_t)Hkv * D;  // elements between consecutive token rows
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const float sl2 = a.scale_log2;

  // This wave's blocks: blk0 + wave + NW*k, k = 0 .. nk-1. Block ids are fetched 64 at a
  // time into one VGPR (lane k holds the id of block k) and broadcast with readlane.
  const int first = blk0 + wave;
  const int nk = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;
  for (int kb = 0; kb < nk; kb += 64) {
    const int jj = first + NW * (kb + lane);
    const int idv = (kb + lane < nk) ? table[jj] : -1;
    const int kend = min(nk - kb, 64);
    for (int k = 0; k < kend; ++k) {
      const int phys = __builtin_amdgcn_readlane(idv, k);
      if (phys < 0 || (int64_t)phys >= a.num_blocks) continue;  // invalid id: never read
      const int jblk = first + NW * (kb + k);
      const uint16_t* kbase = a.k_cache + ((size_t)phys * BS * Hkv + g) * D + col * 8;
      const uint16_t* vbase = a.v_cache + ((size_t)phys * BS * Hkv + g) * D + col * 8;
      uint4 kr[NI], vr[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kr[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)(r0 + RPL * i) * row_stride);
        vr[i] = *reinterpret_cast<const uint4*>(vbase + (size_t)(r0 + RPL * i) * row_stride);
      }
      const int tbase = jblk * BS;
      const bool tail = tbase + BS > tok1;  // block holds positions at or past the end

      float s[G][NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[8];
        unpack8<KT>(kr[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) d = fmaf(qf[h][j], kf[j], d);
          s[h][i] = group_sum<LPR>(d) * sl2;
        }
      }
      if (tail) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bool valid = tbase + r0 + RPL * i < tok1;
#pragma unroll
          for (int h = 0; h < G; ++h) s[h][i] = valid ? s[h][i] : kNegInf;
          if (!valid) vr[i] = make_uint4(0, 0, 0, 0);  // stale rows may hold NaN bits
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mt = s[h][0];
#pragma unroll
        for (int i = 1; i < NI; ++i) mt = fmaxf(mt, s[h][i]);
        const float mn = fmaxf(m[h], mt);
        const float mu = mn == kNegInf ? 0.f : mn;
        const float c = fast_exp2(m[h] - mu);
        l[h] *= c;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= c;
        m[h] = mn;
#pragma unroll
        for (int i = 0; i < NI; ++i) s[h][i] = fast_exp2(s[h][i] - mu);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[8];
        unpack8<KT>(vr[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          l[h] += s[h][i];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(s[h][i], vf[j], acc[h][j]);
        }
      }
    }
  }

  // Merge the RPL row groups of the wave (lanes differing in the bits above log2(LPR)).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mm = m[h];
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) mm = fmaxf(mm, shfl_xor(mm, x));
    const float f = (mm == kNegInf) ? 0.f : fast_exp2(m[h] - mm);
    float lh = l[h] * f;
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) lh += shfl_xor(lh, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = acc[h][j] * f;
#pragma unroll
      for (int x = LPR; x < 64; x <<= 1) v += shfl_xor(v, x);
      acc[h][j] = v;
    }
    m[h] = mm;
    l[h] = lh;
  }

  // Merge the NW waves through LDS, then write the output or the partition's partials.
  __shared__ float sm_m[NW][G], sm_l[NW][G];
  __shared__ float sm_acc[NW][G][D];
  if (r0 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm_acc[wave][h][col * 8 + j] = acc[h][j];
      if (col == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int h = e / D, d = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float num = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(sm_m[w][h] - M);
        num = fmaf(f, sm_acc[w][h][d], num);
        den = fmaf(f, sm_l[w][h], den);
      }
    }
    const size_t row = (size_t)b * Hq + (size_t)g * G + h;
    if (nparts == 1) {
      store_out<OT>(a.out, row * D + d, den > 0.f ? num / den : 0.f);
    } else {
      const size_t pr = row * nparts + part;
      a.ws_acc[pr * D + d] = num;
      if (d == 0) {
        a.ws_ml[pr * 2 + 0] = M;
        a.ws_ml[pr * 2 + 1] = den;
      }
    }
  }
}

template <int D, int G>
static hipError_t launch_dg(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  const unsigned units = (unsigned)((long long)a.batch * a.num_kv_heads * a.nparts);
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    hipLaunchKernelGGL((decode_valu_kernel<D, G, 16, NW, KT, OT>), dim3(units), dim3(NW * 64),
                       0, stream, a);
    return hipGetLastError();
  });
}

bool supported_valu(int head_dim, int group, int block_size) {
  return block_size == 16 && (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 3 || group == 4 || group == 8);
}

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
#define PAGEDKV_CASE(DD, GG) \
  if (a.head_dim == DD && G == GG) return launch_dg<DD, GG>(a, stream);
  PAGEDKV_CASE(128, 1) PAGEDKV_CASE(128, 2) PAGEDKV_CASE(128, 3) PAGEDKV_CASE(128, 4)
  PAGEDKV_CASE(128, 8)
  PAGEDKV_CASE(64, 1) PAGEDKV_CASE(64, 2) PAGEDKV_CASE(64, 3) PAGEDKV_CASE(64, 4)
  PAGEDKV_CASE(64, 8)
#undef PAGEDKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
