// Multi-query causal attention over the paged cache: prefill, chunked prefill and recompute.
//
// Sequence b contributes Q_b query rows, its last Q_b logical positions; query i sits at
// position p = L_b - Q_b + i and attends to positions 0..p through the block table. This is
// the causal attention the Llama engine runs for prefill and recomputation ("vLLM-Style Llama
// Inference Engine with Tensor Parallelism", Features and scope / Implemented; How it works,
// step 4), done over the paged cache as the ragged, padding-free attention over block tables
// that llm-stack's Roadmap plans, with grouped-query heads.
//
// Work decomposition: a workgroup of NW waves takes one KV head g of one sequence and NW*R
// consecutive query tokens; each wave owns R = 16/G tokens x the G query heads of g, i.e. the
// 16 query rows of one MFMA N block. The wave streams the key blocks 0..(its last row's
// position) in pairs, exactly as the decode kernel does (mfma_tiles.h), with a per-lane causal
// mask on the pairs that reach past its first row, and writes its rows normalised.
#include "launch.h"
#include "mfma_tiles.h"

namespace pagedkv {

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
prefill_mfma_kernel(const PrefillArgs a) {
  constexpr int BS = 16;
  constexpr int NCH = D / 32;
  constexpr int EPL = D / 16;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int kg = lane >> 4;

  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int R = 16 / G;  // query tokens per wave
  const int unit = blockIdx.x;
  const int tile = unit % a.ntiles;
  const int g = (unit / a.ntiles) % Hkv;
  const int b = unit / (a.ntiles * Hkv);

  const int q0 = a.cu_seqlens_q[b];
  int Q = a.cu_seqlens_q[b + 1] - q0;
  Q = Q < 0 ? 0 : Q;
  const int tok_base = (tile * NW + wave) * R;  // first query token (in the sequence) of this wave
  if (tok_base >= Q) return;                     // no barriers below: waves are independent
  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);

  const int tok = tok_base + n16 / G;
  const int head = n16 % G;
  const bool row_ok = n16 < R * G && tok < Q;
  const int row_pos = row_ok ? L - Q + tok : -1;  // < 0: no key (only when Q > L)
  const int last_tok = min(tok_base + R, Q) - 1;
  const int p_min = L - Q + tok_base;
  const int p_max = L - Q + last_tok;
  const int tok1 = p_max + 1 > 0 ? p_max + 1 : 0;  // keys 0 .. tok1-1 can matter to this wave
  const int blk1 = (tok1 + BS - 1) / BS;

  bf16x8 qb[NCH];
  {
    const uint16_t* qrow =
        a.q + ((size_t)(q0 + (row_ok ? tok : tok_base)) * Hq + (size_t)g * G + head) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row_ok) w = *reinterpret_cast<const uint4*>(qrow + 32 * c);
      qb[c] = as_bf16x8(w);
    }
  }

  WaveState<EPL> st;
  st.m_run = kNegInf;
  st.l_run = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  PairCtx<D> ctx;
  ctx.k_cache = a.k_cache;
  ctx.v_cache = a.v_cache;
  ctx.table = a.block_tables + (size_t)b * a.max_blocks;
  ctx.row_stride = (size_t)Hkv * D;
  ctx.head_off = (size_t)g * D;
  ctx.num_blocks = a.num_blocks;
  ctx.blk0 = 0;
  ctx.blk1 = blk1;
  ctx.tok1 = tok1;
  ctx.wave = 0;
  ctx.n16 = n16;
  ctx.kg = kg;
  const float sl2 = a.scale_log2;

  // Key pairs (2k, 2k+1), two in flight, loads unconditional (see the decode kernels).
  const int np = (blk1 + 1) / 2;
  if (np > 0) {
    PairTile<NCH, EPL> t[2];
    int2 ids[2];
    ids[0] = pair_ids<D, 1>(ctx, 0);
    ids[1] = pair_ids<D, 1>(ctx, min(1, np - 1));
    pair_load<D, 1>(t[0], ctx, ids[0], 0);
    for (int k = 0; k < np; k += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = k + u;
        const int jl = min(j + 1, np - 1);
        const int ub = (u + 1) % 2;
        pair_load<D, 1>(t[ub], ctx, ids[ub], jl);
        ids[u] = pair_ids<D, 1>(ctx, min(jl + 1, np - 1));
        if (j < np) {
          const int key0 = 2 * BS * j;
          const CausalMask cm{row_pos, key0, key0 + 2 * BS - 1 > p_min};
          pair_compute<NCH, EPL, true>(t[u], st, qb, sl2, kg, cm);
        }
      }
    }
  }

  float l_run = st.l_run;
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* o = a.out + ((size_t)(q0 + tok) * Hq + (size_t)g * G + head) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(o + EPL * (4 * kg + i) + e) =
            make_float4(st.acc[e][i] * inv, st.acc[e + 1][i] * inv, st.acc[e + 2][i] * inv,
                        st.acc[e + 3][i] * inv);
  }
}

bool supported_prefill(int head_dim, int group, int block_size) {
  return block_size == 16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

int prefill_tokens_per_group(int group) { return kWavesPerGroup * (16 / group); }

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  const long long units = (long long)a.batch * a.num_kv_heads * a.ntiles;
  if (a.head_dim == 128)
    hipLaunchKernelGGL((prefill_mfma_kernel<128, NW>), dim3((unsigned)units), dim3(NW * 64), 0,
                       stream, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((prefill_mfma_kernel<64, NW>), dim3((unsigned)units), dim3(NW * 64), 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pagedkv
