// Paged one-token decode attention on the matrix cores (bf16 or fp16 MFMA, fp32 accumulate;
// output in fp32 or in the input format).
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
//   P is split as p = hi + lo with both parts in the input format (bf16: hi = p rounded to
//   nearest even, lo = bf16(p - hi), the exact remainder taken with one v_dot2c_f32_bf16;
//   fp16: both rounded toward zero, weights lifted by 2^7 to stay clear of fp16's small
//   range), two MFMAs per tile, so the weights keep ~16 bits of precision.
// The running max is shared by the four lanes of a head (two cross-lane maxima per step);
// the running sum stays per lane and is reduced once at the end. Waves are merged through
// LDS with the log-sum-exp rule and the result is written out, or left as a partition
// partial for the merge kernel.
#include "decode_step.h"
#include "launch.h"
#include "mfma_tiles.h"

namespace pagedkv {

template <int D, int NW, int KT, int OT, bool ROPE>
__global__ void __launch_bounds__(NW * 64)
decode_mfma_kernel(const DecodeArgs a) {
  constexpr int BS = 16;
  constexpr int NCH = D / 32;  // 32-column chunks of q.K per tile
  constexpr int EPL = D / 16;  // output columns per lane-row in p.V (= p.V MFMAs per step)
  constexpr int DP = D + 4;    // padded LDS row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int kg = lane >> 4;

  const int nparts = a.nparts;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int unit = blockIdx.x;
  const int part = xcd_balanced_part(unit, nparts);
  const int g = (unit / nparts) % Hkv;
  const int b = unit / (nparts * Hkv);

  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int tok0 = part * a.part_tokens;
  if (tok0 >= L && !(L == 0 && part == 0)) {
    if (wave == 0) mark_empty_partition(a, b, g, part, lane);
    return;
  }
  const int tok1 = min(tok0 + a.part_tokens, L);
  const int blk0 = tok0 / BS;
  const int blk1 = (tok1 + BS - 1) / BS;
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;

  // Q^T operand: lane (n16, kg) holds q[head n16][32c + 8kg .. +7] for chunk c (0 if n16>=G).
  uint4 qb[NCH];
  {
    const bool hv = n16 < G;
    const uint16_t* qrow = a.q + ((size_t)b * Hq + (size_t)g * G + (hv ? n16 : 0)) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qb[c] = make_uint4(0, 0, 0, 0);
      if (hv) qb[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
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
  ctx.table = table;
  ctx.row_stride = (size_t)Hkv * D;
  ctx.head_off = (size_t)g * D;
  ctx.num_blocks = a.num_blocks;
  ctx.blk0 = blk0;
  ctx.blk1 = blk1;
  ctx.tok1 = tok1;
  ctx.wave = wave;
  ctx.n16 = n16;
  ctx.kg = kg;
  // Fused step: the new row of this head, loaded unconditionally (from pool slot 0 when there
  // is no step write, then never used) so no memory operation waits behind a branch; the slot
  // is read once, for the position test here and the store at the end.
  const int64_t slot = step_slot(a, b);
  const int sub_pos = step_sub_pos_at(a, slot, table, L);
  NewRow<NCH, EPL> nrow;
  load_new_row(nrow, new_k_row(a, b, g, D), new_v_row(a, b, g, D), n16, kg);
  if constexpr (ROPE)
    rope_pieces<KT>(qb, nrow.k, (float)a.positions[b], a.inv_freq, a.interleaved != 0, kg,
                    lane);
  const float sl2 = a.scale_log2;

  // This wave's block pairs are (blk0 + 2*(wave + NW*k), +1), k = 0 .. np-1. Two pairs are
  // kept in flight: pair k+1's loads are issued before pair k is computed, and block ids are
  // read one pair ahead of the loads. Loads are unconditional (past the last pair they
  // repeat the last pair's addresses, which hit in cache and are never computed), so the
  // loop has no branches around memory operations and the wait counts stay exact.
  const int npairs = (blk1 - blk0 + 1) / 2;
  const int np = wave < npairs ? (npairs - wave + NW - 1) / NW : 0;
  if (np > 0) {
    PairTile<NCH, EPL> t0, t1;
    int2 i0 = pair_ids<D, NW>(ctx, 0);
    int2 i1 = pair_ids<D, NW>(ctx, min(1, np - 1));
    pair_load<D, NW>(t0, ctx, i0, 0);
    for (int k = 0; k < np; k += 2) {
      const int k1 = min(k + 1, np - 1), k2 = min(k + 2, np - 1), k3 = min(k + 3, np - 1);
      pair_load<D, NW>(t1, ctx, i1, k1);
      i0 = pair_ids<D, NW>(ctx, k2);
      use_new_row(t0, nrow, sub_pos, n16, kg);
      pair_compute<KT>(t0, st, qb, sl2, kg);
      pair_load<D, NW>(t0, ctx, i0, k2);
      i1 = pair_ids<D, NW>(ctx, k3);
      if (k + 1 < np) {
        use_new_row(t1, nrow, sub_pos, n16, kg);
        pair_compute<KT>(t1, st, qb, sl2, kg);
      }
    }
  }

  // The step's store comes after every block-table read, so the compiler can keep those reads
  // on the scalar path (no earlier store may have changed the table).
  // It stores from the registers that hold the new rows (rotated key with RoPE), at the slot
  // read above, so it waits on no read.
  if (a.k_new && wave == 0 && (L > 0 ? L - 1 < tok1 : part == 0))
    step_store_regs_at<D>(a, slot, g, nrow, n16, kg);
  if constexpr (ROPE)
    if (wave == 0 && part == 0) store_q_out<D>(a, qb, b, g, G, n16, kg);

  // Sum of the running sums over the four lanes of a head.
  float l_run = st.l_run;
  l_run = row4_sum(l_run);

  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_acc[NW][16][DP];
  if (kg == 0) {
    sm_m[wave][n16] = st.m_run;
    sm_l[wave][n16] = l_run;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_acc[wave][n16][EPL * (4 * kg + i) + e] = st.acc[e][i];
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

// Variant with one wave per KV head: a workgroup of HPW waves takes HPW KV heads of the same
// (sequence, partition), so at any time the workgroup reads HPW*D*2 contiguous bytes of each
// token row of a block instead of D*2, and every wave walks the whole partition on its own
// (no cross-wave merge). Each wave writes its heads' output, or its partition partial for
// the merge kernel.
template <int D, int HPW, int NBUF, int MINW, int KT, int OT, bool ROPE>
__global__ void __launch_bounds__(HPW * 64, MINW)
decode_mfma_hw_kernel(const DecodeArgs a) {
  constexpr int BS = 16;
  constexpr int NCH = D / 32;
  constexpr int EPL = D / 16;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int kg = lane >> 4;

  const int nparts = a.nparts;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int ngrp = (Hkv + HPW - 1) / HPW;
  const int unit = blockIdx.x;
  const int part = xcd_balanced_part(unit, nparts);
  const int hg = (unit / nparts) % ngrp;
  const int b = unit / (nparts * ngrp);
  const int g = hg * HPW + wave;
  if (g >= Hkv) return;  // no barriers below: waves are independent

  // Loads that do not depend on the context length are issued before it arrives: q, the first
  // pair's block ids (every entry of the table row is in bounds to read; entries past the
  // context are ignored below) and, below, that pair's K / V. The wave's start then costs the
  // ids' round trip and the K / V round trip, with the length arriving alongside. The length
  // is read after the pair is issued: a wait for any scalar load waits for all of them, so an
  // earlier read would hold the pair back.
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const int tok0 = part * a.part_tokens;
  const int blk0 = tok0 / BS;
  const int idA0 = blk0 < a.max_blocks ? table[blk0] : -1;
  const int idB0 = blk0 + 1 < a.max_blocks ? table[blk0 + 1] : -1;
  uint4 qb[NCH];
  {
    const bool hv = n16 < G;
    const uint16_t* qrow = a.q + ((size_t)b * Hq + (size_t)g * G + (hv ? n16 : 0)) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qb[c] = make_uint4(0, 0, 0, 0);
      if (hv) qb[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
    }
  }

  PairCtx<D> ctx;
  ctx.k_cache = a.k_cache;
  ctx.v_cache = a.v_cache;
  ctx.table = table;
  ctx.row_stride = (size_t)Hkv * D;
  ctx.head_off = (size_t)g * D;
  ctx.num_blocks = a.num_blocks;
  ctx.blk0 = blk0;
  ctx.wave = 0;
  ctx.n16 = n16;
  ctx.kg = kg;
  // Fused step: the new row of this head, loaded unconditionally (from pool slot 0 when there
  // is no step write, then never used) so no memory operation waits behind a branch; issued
  // before the first pair so that waiting for it never waits for the pair.
  NewRow<NCH, EPL> nrow;
  load_new_row(nrow, new_k_row(a, b, g, D), new_v_row(a, b, g, D), n16, kg);
  const int64_t slot = step_slot(a, b);  // read once: the position test and the store
  // The first pair's K / V loads go out with q's, before the context length arrives: a
  // partition that then turns out empty discards them; every other one saves a round trip.
  PairTile<NCH, EPL> t[NBUF];
  pair_issue(t[0], ctx, make_int2(idA0, idB0), blk0);

  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  if (tok0 >= L && !(L == 0 && part == 0)) {
    // The speculative loads count as used here too, so the compiler keeps them ahead of this
    // branch (and of the wait for the length) instead of sinking them into the main path.
    float neg_inf = kNegInf;
    keep_issued(t[0], neg_inf);
    keep_issued(nrow, neg_inf);
    mark_empty_partition(a, b, g, part, lane, neg_inf);
    return;
  }
  const int tok1 = min(tok0 + a.part_tokens, L);
  const int blk1 = (tok1 + BS - 1) / BS;
  ctx.blk1 = blk1;
  ctx.tok1 = tok1;

  WaveState<EPL> st;
  st.m_run = kNegInf;
  st.l_run = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int sub_pos = step_sub_pos_at(a, slot, table, L);
  if constexpr (ROPE)
    rope_pieces<KT>(qb, nrow.k, (float)a.positions[b], a.inv_freq, a.interleaved != 0, kg,
                    lane);
  const float sl2 = a.scale_log2;

  // Pairs (blk0 + 2k, blk0 + 2k + 1), k = 0 .. np-1, NBUF pairs in flight. Pair j lives in
  // register buffer j % NBUF; the loop is unrolled NBUF times so every buffer index is static.
  // At the step that computes pair j, pair j+NBUF-1 is loaded into the buffer pair j-1 just
  // left, with block ids read one pair ahead of their loads. Past the last pair the loads
  // repeat the last pair's addresses (cache hits, never computed), so no memory operation sits
  // behind a branch and the wait counts stay exact.
  const int np = (blk1 - blk0 + 1) / 2;
  if (np > 0) {
    int2 ids[NBUF];
    ids[0] = make_int2(idA0, blk0 + 1 < blk1 ? idB0 : -1);
    pair_valid(t[0], ctx, ids[0], blk0);  // issued above
#pragma unroll
    for (int u = 1; u < NBUF; ++u) ids[u] = pair_ids<D, 1>(ctx, min(u, np - 1));
#pragma unroll
    for (int u = 1; u < NBUF - 1; ++u) pair_load<D, 1>(t[u], ctx, ids[u], min(u, np - 1));
    for (int k = 0; k < np; k += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int j = k + u;
        const int jl = min(j + NBUF - 1, np - 1);
        const int ub = (u + NBUF - 1) % NBUF;
        pair_load<D, 1>(t[ub], ctx, ids[ub], jl);
        ids[u] = pair_ids<D, 1>(ctx, min(jl + 1, np - 1));
        if (j < np) {
          use_new_row(t[u], nrow, sub_pos, n16, kg);
          pair_compute<KT>(t[u], st, qb, sl2, kg);
        }
      }
    }
  }

  // The step's store comes after every block-table read (see the split-wave kernel), from
  // the registers that hold the new rows, at the slot read above.
  if (a.k_new && (L > 0 ? L - 1 < tok1 : part == 0))
    step_store_regs_at<D>(a, slot, g, nrow, n16, kg);
  if constexpr (ROPE)
    if (part == 0) store_q_out<D>(a, qb, b, g, G, n16, kg);

  float l_run = st.l_run;
  l_run = row4_sum(l_run);
  const bool hv = n16 < G;
  const size_t row0 = (size_t)b * Hq + (size_t)g * G;  // first query head of KV head g
  if (nparts == 1) {
    if (hv) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      const size_t o = (row0 + n16) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          store_out4<OT>(a.out, o + EPL * (4 * kg + i) + e, st.acc[e][i] * inv,
                         st.acc[e + 1][i] * inv, st.acc[e + 2][i] * inv, st.acc[e + 3][i] * inv);
    }
    return;
  }
  // Split: leave this partition's partial (unnormalised output, reference max, sum) for the
  // merge kernel.
  if (hv) {
    const size_t pr = (row0 + n16) * nparts + part;
    float* o = a.ws_acc + pr * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(o + EPL * (4 * kg + i) + e) =
            make_float4(st.acc[e][i], st.acc[e + 1][i], st.acc[e + 2][i], st.acc[e + 3][i]);
    if (kg == 0) {
      a.ws_ml[pr * 2 + 0] = st.m_run;
      a.ws_ml[pr * 2 + 1] = l_run;
    }
  }
}

bool supported_mfma(int head_dim, int group, int block_size) {
  return block_size == 16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  const unsigned units = (unsigned)((long long)a.batch * a.num_kv_heads * a.nparts);
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    constexpr bool kRope = KT == kDtBf16;  // bf16 inputs only, as in the head-per-wave launch
    const bool rope = a.positions != nullptr;
    if (rope && !kRope) return hipErrorInvalidValue;
    if (a.head_dim == 128 && rope)
      hipLaunchKernelGGL((decode_mfma_kernel<128, NW, KT, OT, kRope>), dim3(units), dim3(NW * 64),
                         0, stream, a);
    else if (a.head_dim == 128)
      hipLaunchKernelGGL((decode_mfma_kernel<128, NW, KT, OT, false>), dim3(units),
                         dim3(NW * 64), 0, stream, a);
    else if (a.head_dim == 64 && rope)
      hipLaunchKernelGGL((decode_mfma_kernel<64, NW, KT, OT, kRope>), dim3(units), dim3(NW * 64),
                         0, stream, a);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL((decode_mfma_kernel<64, NW, KT, OT, false>), dim3(units), dim3(NW * 64),
                         0, stream, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  });
}

hipError_t launch_decode_mfma_hw(const DecodeArgs& a, hipStream_t stream) {
  constexpr int HPW = kHeadsPerGroup;
  // Two block pairs in flight per wave. Three or four (which need occupancy 1) measured
  // slower on the cold 2 x 32768 case (52-53 us against 49), and no faster elsewhere; two
  // keep two waves per SIMD.
  constexpr int NBUF = 2;
  const long long ngrp = (a.num_kv_heads + HPW - 1) / HPW;
  const unsigned units = (unsigned)((long long)a.batch * ngrp * a.nparts);
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    // The rotary step takes bf16 inputs only (the host layer checks): no fp16 instance.
    constexpr bool kRope = KT == kDtBf16;
    const bool rope = a.positions != nullptr;
    if (rope && !kRope) return hipErrorInvalidValue;
    if (a.head_dim == 128 && rope)
      hipLaunchKernelGGL((decode_mfma_hw_kernel<128, HPW, NBUF, 2, KT, OT, kRope>), dim3(units),
                         dim3(HPW * 64), 0, stream, a);
    else if (a.head_dim == 128)
      hipLaunchKernelGGL((decode_mfma_hw_kernel<128, HPW, NBUF, 2, KT, OT, false>), dim3(units),
                         dim3(HPW * 64), 0, stream, a);
    else if (a.head_dim == 64 && rope)
      hipLaunchKernelGGL((decode_mfma_hw_kernel<64, HPW, NBUF, 2, KT, OT, kRope>), dim3(units),
                         dim3(HPW * 64), 0, stream, a);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL((decode_mfma_hw_kernel<64, HPW, NBUF, 2, KT, OT, false>), dim3(units),
                         dim3(HPW * 64), 0, stream, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  });
}

}  // namespace pagedkv
