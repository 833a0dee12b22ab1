// Paged one-token decode attention on the matrix cores (bf16 MFMA, fp32 accumulate).
//
// Same computation as the vector-ALU kernel: for every sequence b and query head h,
// softmax(scale * q[b,h] . K^T) V over the context_lens[b] positions read through
// block_tables[b] (mini-vLLM README, paged KV-cache paragraph; "vLLM-Style Llama Inference
// Engine with Tensor Parallelism", How it works, step 4), grouped-query heads packed per KV
// head, online softmax with fp32 accumulation (llm-stack, Attention kernel section).
//
// Why the matrix cores: per token and KV head the G packed query heads need G*D multiply-adds
// for q.K and G*D for p*V against 4*D bytes of K and V, which is ~1 flop/byte per query head.
// In fp32 vector code that, plus the bf16 unpacking and the cross-lane reductions, keeps the
// vector ALU busy a large fraction of the time while HBM streams. Both products are small
// dense contractions (a 16-token tile against the G query rows), so they map onto
// v_mfma_f32_16x16x32_bf16 with the G heads padded to 16 columns. The padding wastes matrix
// throughput that this HBM-bound loop has in excess, and it frees the vector ALU.
//
// One wave handles a pair of 16-token blocks (32 tokens) per step:
//   S^T = K_tile . Q^T   M = 16 tokens, N = 16 head slots (G used), K = 32 columns of D per
//                        MFMA. A lane (n = lane%16, kg = lane/16) feeds 8 consecutive bf16
//                        of row n straight from global memory (16-byte loads), and the Q
//                        slice of head n with the same columns. The result leaves lane
//                        (n, kg) holding scores of tokens 4kg..4kg+3 for head n.
//   O^T += V^T . P^T     M = 16 output columns (d = EPL*m + e for MFMA e), N = 16 head slots,
//                        K = 32 tokens. The contraction order of tokens is free, so token
//                        slot (kg, j) is taken to be the token whose score lane (n, kg)
//                        already holds (j<4: first block, row 4kg+j; j>=4: second block,
//                        row 4kg+j-4). P^T is then built in place with no data movement;
//                        V^T needs 8 token rows per lane, loaded as EPL contiguous bf16 per
//                        row and transposed in registers with v_perm_b32.
//   P is split as p = hi + lo with both parts in bf16 (hi = p truncated to bf16, exact;
//   lo = bf16(p - hi)), two MFMAs per tile, so the weights keep ~16 bits of precision.
// The running max is shared by the four lanes of a head (two cross-lane maxima per step);
// the running sum stays per lane and is reduced once at the end. Waves are merged through
// LDS with the log-sum-exp rule and the result is written out, or left as a partition
// partial for the merge kernel.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& w) {
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b,
                                                const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Low / high bf16 halves of two words packed into one word (x's half first).
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Row of EPL consecutive bf16 values (EPL = 8: 16 bytes, EPL = 4: 8 bytes).
template <int EPL> struct VRow;
template <> struct VRow<8> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void keep_if(bool v) {
    w.x = v ? w.x : 0u; w.y = v ? w.y : 0u; w.z = v ? w.z : 0u; w.w = v ? w.w : 0u;
  }
  __device__ __forceinline__ uint32_t word(int i) const {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
  }
};
template <> struct VRow<4> {
  uint2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void keep_if(bool v) { w.x = v ? w.x : 0u; w.y = v ? w.y : 0u; }
  __device__ __forceinline__ uint32_t word(int i) const { return i == 0 ? w.x : w.y; }
};

// Slack of the lazily updated softmax reference max, in log2 units (weights <= 2^8).
constexpr float kRescaleSlack = 8.f;

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
decode_mfma_kernel(const DecodeArgs a) {
  constexpr int BS = 16;
  constexpr int NCH = D / 32;  // 32-column chunks of q.K per tile
  constexpr int EPL = D / 16;  // output columns per lane-row in P.V (= PV MFMAs per step)
  constexpr int DP = D + 4;    // padded LDS row

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int kg = lane >> 4;

  const int nparts = a.nparts;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int unit = blockIdx.x;
  const int part = unit % nparts;
  const int g = (unit / nparts) % Hkv;
  const int b = unit / (nparts * Hkv);

  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int tok0 = part * a.part_tokens;
  if (tok0 >= L && !(L == 0 && part == 0)) return;
  const int tok1 = min(tok0 + a.part_tokens, L);
  const int blk0 = tok0 / BS;
  const int blk1 = (tok1 + BS - 1) / BS;

  // Q^T operand: lane (n16, kg) holds q[head n16][32c + 8kg .. +7] for chunk c (0 if n16>=G).
  bf16x8 qb[NCH];
  {
    const bool hv = n16 < G;
    const uint16_t* qrow = a.q + ((size_t)b * Hq + (size_t)g * G + (hv ? n16 : 0)) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (hv) w = *reinterpret_cast<const uint4*>(qrow + 32 * c);
      qb[c] = as_bf16x8(w);
    }
  }

  float m_run = kNegInf;  // running max of head n16 (log2 units), equal across kg
  float l_run = 0.f;      // this lane's share of the running sum
  floatx4 acc[EPL];       // O^T: acc[e][i] = out[head n16][EPL*(4kg+i) + e]
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row_stride = (size_t)Hkv * D;
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const float sl2 = a.scale_log2;

  // This wave's block pairs: (blk0 + 2*(wave + NW*k), +1), k = 0 .. np-1. Ids are fetched
  // 64 pairs at a time (lane k holds pair k's two ids) and broadcast with readlane.
  const int nblk = blk1 - blk0;
  const int npairs = (nblk + 1) / 2;
  const int np = wave < npairs ? (npairs - wave + NW - 1) / NW : 0;
  for (int kb = 0; kb < np; kb += 64) {
    int idA = -1, idB = -1;
    {
      const int jA = blk0 + 2 * (wave + NW * (kb + lane));
      if (kb + lane < np) {
        idA = table[jA];
        if (jA + 1 < blk1) idB = table[jA + 1];
      }
    }
    const int kend = min(np - kb, 64);
    for (int k = 0; k < kend; ++k) {
      const int jA = blk0 + 2 * (wave + NW * (kb + k));
      int pA = __builtin_amdgcn_readlane(idA, k);
      int pB = __builtin_amdgcn_readlane(idB, k);
      const bool okA = pA >= 0 && (int64_t)pA < a.num_blocks;
      const bool okB = pB >= 0 && (int64_t)pB < a.num_blocks;
      // An invalid or absent block is replaced by block 0 (always in the pool) and all of its
      // tokens are masked below, so its contents never reach the result.
      const int tA = jA * BS, tB = tA + BS;
      const int lastA = okA ? min(tok1 - tA, BS) : 0;  // valid rows in each block
      const int lastB = okB ? min(tok1 - tB, BS) : 0;
      pA = okA ? pA : 0;
      pB = okB ? pB : 0;

      const uint16_t* kA = a.k_cache + ((size_t)pA * BS * Hkv + g) * D;
      const uint16_t* kB = a.k_cache + ((size_t)pB * BS * Hkv + g) * D;
      const uint16_t* vA = a.v_cache + ((size_t)pA * BS * Hkv + g) * D;
      const uint16_t* vB = a.v_cache + ((size_t)pB * BS * Hkv + g) * D;

      uint4 ka[NCH], kbv[NCH];
      VRow<EPL> vr[8];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        ka[c] = *reinterpret_cast<const uint4*>(kA + (size_t)n16 * row_stride + 32 * c + 8 * kg);
        kbv[c] = *reinterpret_cast<const uint4*>(kB + (size_t)n16 * row_stride + 32 * c + 8 * kg);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vr[j].load(vA + (size_t)(4 * kg + j) * row_stride + EPL * n16);
        vr[4 + j].load(vB + (size_t)(4 * kg + j) * row_stride + EPL * n16);
      }

      floatx4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        sA = mfma16x16x32(as_bf16x8(ka[c]), qb[c], sA);
        sB = mfma16x16x32(as_bf16x8(kbv[c]), qb[c], sB);
      }
      float s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sA[i] * sl2;
        s[4 + i] = sB[i] * sl2;
      }
      if (lastA < BS || lastB < BS) {  // a block holds positions at or past the end
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool va = 4 * kg + i < lastA;
          const bool vb = 4 * kg + i < lastB;
          s[i] = va ? s[i] : kNegInf;
          s[4 + i] = vb ? s[4 + i] : kNegInf;
          vr[i].keep_if(va);  // stale rows may hold NaN bits; 0 * NaN would poison P.V
          vr[4 + i].keep_if(vb);
        }
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      // Lazy rescaling: the reference max moves only when a score exceeds it by more than
      // kRescaleSlack (log2 units), so weights stay <= 2^kRescaleSlack and the accumulator is
      // rescaled on few steps instead of every step. Any reference value gives the same
      // softmax; the final normalisation divides it out.
      const float mn = fmaxf(m_run, mx);
      const bool upd = mn > m_run + kRescaleSlack;  // also true while m_run is -inf
      if (__any(upd)) {
        const float m_new = upd ? mn : m_run;
        const float alpha = upd ? fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new)) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float mu = m_run == kNegInf ? 0.f : m_run;
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(s[i] - mu);
        psum += p[i];
      }
      l_run += psum;

      // P^T operand, split into bf16 hi (truncation, exact) + bf16 lo (rounded remainder).
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t u0 = __float_as_uint(p[2 * t]), u1 = __float_as_uint(p[2 * t + 1]);
        hw[t] = pack_hi(u0, u1);
        const float r0 = p[2 * t] - __uint_as_float(u0 & 0xffff0000u);
        const float r1 = p[2 * t + 1] - __uint_as_float(u1 & 0xffff0000u);
        const __bf16 b0 = (__bf16)r0, b1 = (__bf16)r1;
        lw[t] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      }
      const bf16x8 phi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 plo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));

      // V^T operand for output column set e: 8 token slots of column EPL*n16 + e.
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t x = vr[2 * t].word(e / 2), y = vr[2 * t + 1].word(e / 2);
          w[t] = (e & 1) ? pack_hi(x, y) : pack_lo(x, y);
        }
        const bf16x8 vt = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        acc[e] = mfma16x16x32(vt, phi, acc[e]);
        acc[e] = mfma16x16x32(vt, plo, acc[e]);
      }
    }
  }

  // Sum of the running sums over the four lanes of a head.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);

  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_acc[NW][16][DP];
  if (kg == 0) {
    sm_m[wave][n16] = m_run;
    sm_l[wave][n16] = l_run;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_acc[wave][n16][EPL * (4 * kg + i) + e] = acc[e][i];
  __syncthreads();

  for (int x = threadIdx.x; x < G * D; x += NW * 64) {
    const int h = x / D, d = x % D;
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
      a.out[row * D + d] = den > 0.f ? num / den : 0.f;
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

bool supported_mfma(int head_dim, int group, int block_size) {
  return block_size == 16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  const long long units = (long long)a.batch * a.num_kv_heads * a.nparts;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<128, NW>), dim3((unsigned)units), dim3(NW * 64), 0,
                       stream, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<64, NW>), dim3((unsigned)units), dim3(NW * 64), 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pagedkv
