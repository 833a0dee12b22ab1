// Paged decode attention for batches of many sequences of uneven length: a persistent,
// evenly divided ("stream-K") walk over the batch's work on the matrix cores.
//
// The computation is that of the other decode kernels: for every sequence b and query head h,
// softmax(scale * q[b,h] . K^T) V over the context_lens[b] positions read through
// block_tables[b] (mini-vLLM README, paged KV-cache paragraph: sequences of very different
// lengths share one block pool; "vLLM-Style Llama Inference Engine with Tensor Parallelism",
// How it works, step 4), with the tiles, the online softmax and the fused step of the
// head-per-wave kernel (mfma_tiles.h, decode_step.h).
//
// Why another decomposition: with a fixed partition size, a ragged batch leaves many
// (sequence, partition) units empty and others full, so some compute units idle from the start
// while the full partitions, each streamed by one workgroup at that workgroup's own bandwidth,
// set the time. Here the work is counted on the device and cut into equal slices:
//   items = (sequence b, group of HPW KV heads, pair k of 32 tokens), b-major, then the head
//   group, then k; sequence b holds ngrp * ceil(L_b / 32) items, W in all.
// Workgroup w of N (one per compute unit: a second resident workgroup's loads were served
// after most of the first one's, and it finished a quarter of the dispatch later) takes the
// slice [start(w), start(w+1)) of the items: equal slices of q = max(min_pairs, ceil(W / N)),
// or on the whole device slices weighted by the XCD the workgroup runs on (SkDivision below);
// each of its HPW waves streams one KV head of those items. Where the slice crosses from one
// (sequence, head group) to the next, the wave closes the first as a segment and starts the
// next: each segment leaves a partial softmax result (unnormalised output, reference max, sum)
// in slot j = w - (first workgroup of that (sequence, head group)) of the split workspace, and
// the workgroup that closes the last segment of a (sequence, head group) marks its remaining
// slots empty. Every slot is therefore written on every call, and the partition merge (the
// log-sum-exp rule of decode_reduce.hip) combines them. Every slice holds at least min_pairs
// items, which bounds the slots a (sequence, head group) of at most pairs_max pairs can need:
// (pairs_max - 1) / min_pairs + 2.
// Sequences of length 0 hold no items; workgroup b mod N marks their slots and does their
// part of the fused step.
#include "decode_step.h"
#include "launch.h"
#include "mfma_tiles.h"

namespace pagedkv {

// Pairs in flight per wave (three measured 3% slower than two on the ragged and the uniform
// long batches), and the least waves per SIMD the registers are sized for (the grid holds
// one workgroup per compute unit, one wave per SIMD).
#ifndef PAGEDKV_STREAM_NBUF
#define PAGEDKV_STREAM_NBUF 2
#endif
#ifndef PAGEDKV_STREAM_MINW
#define PAGEDKV_STREAM_MINW 1
#endif

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan_i32(int v, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int u = __shfl_up(v, s, 64);
    if (lane >= s) v += u;
  }
  return v;
}

__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

// Marks slots [s0, nparts) of KV head g's G query rows of sequence b as holding no keys.
__device__ __forceinline__ void mark_slots_empty(const DecodeArgs& a, int b, int g, int s0,
                                                 int i) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (i >= G) return;
  const size_t row = (size_t)b * a.num_q_heads + (size_t)g * G + i;
  for (int s = s0; s < a.nparts; ++s) {
    a.ws_ml[(row * a.nparts + s) * 2 + 0] = kNegInf;
    a.ws_ml[(row * a.nparts + s) * 2 + 1] = 0.f;
  }
}

// A pair of a workgroup's slice: pair k of (sequence b, head group hg), in the segment of pairs
// k0 .. kend - 1 of (b, hg) that the slice holds. S: first item of sequence b; first: first item
// of (b, hg). All wave-uniform.
struct SkPos {
  int b, S, hg, L, pairs, k, k0, kend, first;
};

// The division of the batch's W items among the N workgroups: slice v is [start(v), start(v+1)).
// Uniform: slices of q = max(min_pairs, ceil(W / N)) items. XCD-weighted: the dispatcher deals
// workgroup v to XCD v mod 8, and on MI355X the odd-numbered XCDs stream about 2.8% slower than
// the even ones (per-workgroup wall-clock stamps of this kernel on three parts, for pools
// allocated in different places, two seeds and a ragged batch; the same on each). Slices then
// get the weights kSkEven and kSkOdd by v's parity, start(v) = round(W c(v) / c(N)) with c(v) the
// weight of workgroups 0 .. v-1, so that every XCD finishes at about the same time (each slice
// within one item of its share: on the 64 x 8192 batch 130 and 126 items instead of 128). They
// are used only when even an odd slice keeps at least min_pairs items, which keeps the planned
// number of partial slots sufficient.
constexpr int kSkEven = 507, kSkOdd = 493;
struct SkDivision {
  int W, N, q;
  bool weighted;
  long long cN;
  __device__ __forceinline__ static long long c(int v) {
    return (long long)(v >> 1) * (kSkEven + kSkOdd) + (v & 1) * kSkEven;
  }
  __device__ __forceinline__ void init(int W_, int N_, int min_pairs, bool xcd) {
    W = W_;
    N = N_;
    q = max(min_pairs, (W + N - 1) / N);
    cN = c(N);
    weighted = xcd && (long long)W * kSkOdd >= (long long)(min_pairs + 1) * cN;
  }
  __device__ __forceinline__ int start(int v) const {
    return weighted ? (int)(((long long)W * c(v) + cN / 2) / cN)
                    : (int)min((long long)v * q, (long long)W);
  }
  // The slice holding item x (0 <= x < W).
  __device__ __forceinline__ int slice_of(int x) const {
    if (!weighted) return x / q;
    int v = (int)((long long)x * N / W);
    while (v + 1 < N && start(v + 1) <= x) ++v;
    while (v > 0 && start(v) > x) --v;
    return v;
  }
};

// The fused step's facts of a segment, read ahead with its first pair's block ids: the new
// token's slot (-1 when the segment does not end its sequence, or without new rows), the block
// table's entry for position L - 1, and with RoPE the sequence's position.
struct SegFacts {
  int64_t slot;
  int entry;
  float pos;
};

// One wave's K / V tile of pair p for KV head g: the context a pair load needs.
template <int D>
__device__ __forceinline__ PairCtx<D> sk_ctx(const DecodeArgs& a, const int32_t* tables,
                                             const SkPos& p, int g, int n16, int kg) {
  PairCtx<D> c;
  c.k_cache = a.k_cache;
  c.v_cache = a.v_cache;
  c.table = tables + (size_t)p.b * a.max_blocks;
  c.row_stride = (size_t)a.num_kv_heads * D;
  c.head_off = (size_t)g * D;
  c.num_blocks = a.num_blocks;
  c.blk0 = 0;
  c.blk1 = (p.L + 15) / 16;  // blocks of the sequence; a pair never crosses a segment
  c.tok1 = p.L;
  c.wave = 0;
  c.n16 = n16;
  c.kg = kg;
  return c;
}

// Block ids of pair p (scalar loads; both blocks of the pair lie before blk1 or are absent).
template <int D>
__device__ __forceinline__ int2 sk_ids(const PairCtx<D>& c, const SkPos& p) {
  const int jA = 2 * p.k;
  return make_int2(c.table[jA], jA + 1 < c.blk1 ? c.table[jA + 1] : -1);
}

// Writes the partial of the segment that ends with pair p (slot w - slice_of(first)) and, when it
// ends its (sequence, head group), marks that sequence's remaining slots empty; with RoPE the
// segment that starts the sequence stores the rotated q. (The step's new rows are stored by
// the kernel's loop when the segment's last pair is scored.)
template <int D, int NCH, int EPL, bool ROPE>
__device__ __forceinline__ void sk_close(const DecodeArgs& a, const SkPos& p, int g, int slot,
                                         const WaveState<EPL>& st, const uint4 (&qb)[NCH],
                                         int lane) {
  const int n16 = lane & 15, kg = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool last = p.kend == p.pairs;
  if constexpr (ROPE)
    if (p.k0 == 0) store_q_out<D>(a, qb, p.b, g, G, n16, kg);
  const float l_run = row4_sum(st.l_run);
  const size_t row0 = (size_t)p.b * a.num_q_heads + (size_t)g * G;
  if (n16 < G) {
    const size_t pr = (row0 + n16) * a.nparts + slot;
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
  if (last && kg == 0) mark_slots_empty(a, p.b, g, slot + 1, n16);
}

// A sequence of length 0: no keys (every slot empty), and its share of the fused step: the new
// rows stored at its slot, and with RoPE its rotated q (the other kernels do this in
// partition 0).
template <int D, int KT, bool ROPE>
__device__ __forceinline__ void sk_empty_sequence(const DecodeArgs& a, const int64_t* slots,
                                                  const int32_t* positions, int b, int g,
                                                  int lane) {
  constexpr int NCH = D / 32;
  constexpr int EPL = D / 16;
  const int n16 = lane & 15, kg = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  if (kg == 0) mark_slots_empty(a, b, g, 0, n16);
  if (!a.k_new) return;
  if constexpr (ROPE) {
    uint4 qb[NCH];
    const bool hv = n16 < G;
    const uint16_t* qrow =
        a.q + ((size_t)b * a.num_q_heads + (size_t)g * G + (hv ? n16 : 0)) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) qb[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
    NewRow<NCH, EPL> nrow;
    load_new_row(nrow, new_k_row(a, b, g, D), new_v_row(a, b, g, D), n16, kg);
    rope_pieces<KT>(qb, nrow.k, (float)positions[b], a.inv_freq, a.interleaved != 0, kg,
                    lane);
    step_store_regs<D>(a, slots, b, g, nrow, n16, kg);
    store_q_out<D>(a, qb, b, g, G, n16, kg);
  } else {
    step_store<D>(a, slots, b, g, lane);
  }
}

// The block tables, context lengths, slot mapping and positions come as separate,
// restrict-qualified arguments: this kernel stores partials between segments, and only a
// read-only pointer the compiler knows no store can reach keeps these uniform reads on the
// scalar path (a vector load there would make the loop's waits count it with the key / value
// loads and serialise the pipeline).
template <int D, int HPW, int NBUF, int MINW, int KT, int OT, bool ROPE>
__global__ void __launch_bounds__(HPW * 64, MINW)
decode_mfma_sk_kernel(const DecodeArgs a, const int32_t* __restrict__ tables,
                      const int32_t* __restrict__ lens, const int64_t* __restrict__ slots,
                      const int32_t* __restrict__ positions) {
  static_assert(NBUF == 2 || NBUF == 3, "two or three pairs in flight");
  constexpr int BS = 16, PT = 2 * BS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int B = a.batch, Hkv = a.num_kv_heads;
  const int ngrp = (Hkv + HPW - 1) / HPW;
  const int Lmax = a.max_blocks * BS;
  const int N = gridDim.x, w = blockIdx.x;

  constexpr int NCH = D / 32;
  constexpr int EPL = D / 16;
  const int n16 = lane & 15, kg = lane >> 4;
  const int Hq = a.num_q_heads, G = Hq / Hkv;
  uint4 qb[NCH];
  NewRow<NCH, EPL> nrow;
  const auto load_q = [&](int b, int g) {
    const bool hv = n16 < G;
    const uint16_t* qrow = a.q + ((size_t)b * Hq + (size_t)g * G + (hv ? n16 : 0)) * D + 8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qb[c] = make_uint4(0, 0, 0, 0);
      if (hv) qb[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
    }
    load_new_row(nrow, new_k_row(a, b, g, D), new_v_row(a, b, g, D), n16, kg);
  };

  // Lengths: lane l holds sequence l's (of the first 64), read once; the total work needs all.
  int Lv = 0, mine = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int L = c0 + lane < B ? clamp_len(lens[c0 + lane], Lmax) : 0;
    if (c0 == 0) Lv = L;
    mine += (L + PT - 1) / PT;
  }
  const auto len_of = [&](int b) {  // b uniform
    return b < 64 ? __builtin_amdgcn_readlane(Lv, b) : clamp_len(lens[b], Lmax);
  };
  const int W = __builtin_amdgcn_readfirstlane(wave_sum_i32(mine)) * ngrp;
  SkDivision dv;
  dv.init(W, N, a.sk_min_pairs, a.sk_xcd_weights != 0);
  const int lo = dv.start(w), hi = dv.start(w + 1);
  if (lo < hi) {
    // The sequence holding item lo, and the first item of that sequence: a scan of the items
    // per sequence, 64 sequences at a time.
    int b0 = 0, S0 = 0;
    {
      int base = 0;
      for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int L = c0 == 0 ? Lv : (bb < B ? clamp_len(lens[bb], Lmax) : 0);
        const int cb = (L + PT - 1) / PT * ngrp;
        const int incl = wave_scan_i32(cb, lane) + base;
        const unsigned long long hit = __ballot(cb > 0 && incl - cb <= lo && lo < incl);
        if (hit) {
          const int l = __ffsll((long long)hit) - 1;
          b0 = c0 + l;
          S0 = __shfl(incl - cb, l, 64);
          break;
        }
        base = __shfl(incl, 63, 64);
      }
    }
    // The pair at item `item` of the slice, searching forward from sequence b (first item S).
    const auto pos_at = [&](int item, int b, int S) {
      SkPos p;
      for (;;) {
        const int L = len_of(b);
        const int pairs = (L + PT - 1) / PT;
        if (item < S + pairs * ngrp) {
          p.b = b;
          p.S = S;
          p.L = L;
          p.pairs = pairs;
          p.hg = (item - S) / pairs;
          p.first = S + p.hg * pairs;
          p.k = p.k0 = item - p.first;
          p.kend = min(hi, p.first + pairs) - p.first;
          return p;
        }
        S += pairs * ngrp;  // past this sequence (or it is empty): the next one
        ++b;
      }
    };
    // The pair after p in the slice; past the slice's end, p itself (its loads then repeat).
    const auto pos_next = [&](const SkPos& p) {
      if (p.k + 1 < p.kend) {
        SkPos n = p;
        ++n.k;
        return n;
      }
      return p.first + p.kend < hi ? pos_at(p.first + p.kend, p.b, p.S) : p;
    };
    const auto head = [&](const SkPos& p) { return p.hg * HPW + wave; };
    const auto head_ld = [&](const SkPos& p) { return min(head(p), Hkv - 1); };
    const auto load_ids = [&](const SkPos& p) {
      return sk_ids<D>(sk_ctx<D>(a, tables, p, head_ld(p), n16, kg), p);
    };
    // The fused step's facts of the segment that pair p starts, read with p's block ids, NBUF
    // pairs before p is computed, so that neither the segment's start nor its close waits on a
    // read of its own: with RoPE the position; for the segment that ends its sequence, the new
    // token's slot and the table's entry for position L - 1.
    const auto seg_facts = [&](const SkPos& p) {
      SegFacts f{-1, 0, 0.f};
      if (p.k == p.k0) {
        if (a.k_new && p.kend == p.pairs) {
          f.slot = slots[p.b];
          f.entry = tables[(size_t)p.b * a.max_blocks + (p.L - 1) / BS];
        }
        if constexpr (ROPE) f.pos = (float)positions[p.b];
      }
      return f;
    };

    // One continuous pipeline over the slice's pairs, across segment boundaries: pair j is
    // computed from buffer j % NBUF while pairs j + 1 .. j + NBUF - 1 are in flight in the
    // others, with block ids read one pair further ahead, as in the head-per-wave kernel. When
    // pair j ends a segment, the next segment's q and new rows are loaded right after pair j's
    // scores (q is not needed again), and its first pairs are already in flight, so the
    // boundary costs no round trip. pp[0] is the pair computed next, pp[i] the i-th after it;
    // ids[i] and sf[i] hold pp[i]'s block ids and segment facts.
    SkPos pp[NBUF + 1];
    pp[0] = pos_at(lo, __builtin_amdgcn_readfirstlane(b0), __builtin_amdgcn_readfirstlane(S0));
#pragma unroll
    for (int i = 1; i <= NBUF; ++i) pp[i] = pos_next(pp[i - 1]);
    PairTile<NCH, EPL> t[NBUF];
    int2 ids[NBUF];
    SegFacts sf[NBUF];
    ids[0] = load_ids(pp[0]);
    sf[0] = seg_facts(pp[0]);
    load_q(pp[0].b, head_ld(pp[0]));
#pragma unroll
    for (int i = 1; i < NBUF; ++i) {
      ids[i] = load_ids(pp[i]);
      sf[i] = seg_facts(pp[i]);
    }
    const int P = hi - lo;
#pragma unroll
    for (int i = 0; i + 1 < NBUF; ++i) {  // past the slice's end: pair 0's addresses again
      const SkPos& pi = i < P ? pp[i] : pp[0];
      const PairCtx<D> c = sk_ctx<D>(a, tables, pi, head_ld(pi), n16, kg);
      const int2 ii = i < P ? ids[i] : ids[0];
      pair_issue(t[i], c, ii, 2 * pi.k);
      pair_valid(t[i], c, ii, 2 * pi.k);
    }
    WaveState<EPL> st;
    int sub_pos = -1;
    int64_t seg_slot = -1;  // the current segment's new-token slot (-1: it stores nothing)
    const float sl2 = a.scale_log2;
    for (int j = 0; j < P; j += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int jj = j + u;
        // Issue pair jj + NBUF - 1 (past the end: repeat pair jj's addresses, never computed).
        {
          const bool more = jj + NBUF - 1 < P;
          const SkPos& pi = more ? pp[NBUF - 1] : pp[0];
          const int2 ii = more ? ids[NBUF - 1] : ids[0];
          const PairCtx<D> c = sk_ctx<D>(a, tables, pi, head_ld(pi), n16, kg);
          pair_issue(t[(u + NBUF - 1) % NBUF], c, ii, 2 * pi.k);
          pair_valid(t[(u + NBUF - 1) % NBUF], c, ii, 2 * pi.k);
        }
        const int2 idn = load_ids(pp[NBUF]);
        const SegFacts sfn = seg_facts(pp[NBUF]);
        const SkPos& pc = pp[0];
        if (jj < P) {
          if (pc.k == pc.k0) {  // the segment starts: fresh state
            st.m_run = kNegInf;
            st.l_run = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) st.acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
            seg_slot = sf[0].slot;
            sub_pos = sub_pos_of(a, sf[0].slot, sf[0].entry, pc.L);
            if constexpr (ROPE)
              rope_pieces<KT>(qb, nrow.k, sf[0].pos, a.inv_freq, a.interleaved != 0, kg, lane);
          }
          use_new_row(t[u], nrow, sub_pos, n16, kg);
          float sc[8];
          pair_scores<KT>(t[u], qb, sl2, sc);
          const bool closes = pc.k + 1 == pc.kend;
          // The sequence's last segment stores the step's new rows from registers (as loaded,
          // or the rotated key), at the slot read with its first pair, before the next
          // segment's loads replace them.
          if (closes && pc.kend == pc.pairs && head(pc) < Hkv)
            step_store_regs_at<D>(a, seg_slot, head(pc), nrow, n16, kg);
          // Without RoPE, q and the new row are dead once the closing pair's scores are taken:
          // the next segment's load right away. With RoPE the close stores them (rotated), so
          // they load after it.
          if constexpr (!ROPE)
            if (closes && jj + 1 < P) load_q(pp[1].b, head_ld(pp[1]));
          pair_finish<KT>(t[u], st, sc, kg);
          if (closes) {
            const int g = head(pc);
            if (g < Hkv)
              sk_close<D, NCH, EPL, ROPE>(a, pc, g, w - dv.slice_of(pc.first), st, qb, lane);
            if constexpr (ROPE)
              if (jj + 1 < P) load_q(pp[1].b, head_ld(pp[1]));
          }
        }
#pragma unroll
        for (int i = 0; i < NBUF; ++i) pp[i] = pp[i + 1];
        pp[NBUF] = pos_next(pp[NBUF]);
#pragma unroll
        for (int i = 0; i + 1 < NBUF; ++i) {
          ids[i] = ids[i + 1];
          sf[i] = sf[i + 1];
        }
        ids[NBUF - 1] = idn;
        sf[NBUF - 1] = sfn;
      }
    }
  }

  // Sequences of length 0 (no items): workgroup b mod N does their share.
  for (int b = w; b < B; b += N)
    if (len_of(b) == 0)
      for (int hg = 0; hg < ngrp; ++hg)
        if (hg * HPW + wave < Hkv) sk_empty_sequence<D, KT, ROPE>(a, slots, positions, b, hg * HPW + wave,
                                                             lane);
}

hipError_t launch_decode_mfma_sk(const DecodeArgs& a, int workgroups, hipStream_t stream) {
  constexpr int HPW = kHeadsPerGroup;
  constexpr int NBUF = PAGEDKV_STREAM_NBUF;
  constexpr int MINW = PAGEDKV_STREAM_MINW;
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    constexpr bool kRope = KT == kDtBf16;  // bf16 inputs only, as in the other launches
    const bool rope = a.positions != nullptr;
    if (rope && !kRope) return hipErrorInvalidValue;
    const dim3 grid(workgroups), block(HPW * 64);
    if (a.head_dim == 128 && rope)
      hipLaunchKernelGGL((decode_mfma_sk_kernel<128, HPW, NBUF, MINW, KT, OT, kRope>), grid, block,
                         0, stream, a, a.block_tables, a.context_lens, a.slot_mapping,
                         a.positions);
    else if (a.head_dim == 128)
      hipLaunchKernelGGL((decode_mfma_sk_kernel<128, HPW, NBUF, MINW, KT, OT, false>), grid, block,
                         0, stream, a, a.block_tables, a.context_lens, a.slot_mapping,
                         a.positions);
    else if (a.head_dim == 64 && rope)
      hipLaunchKernelGGL((decode_mfma_sk_kernel<64, HPW, NBUF, MINW, KT, OT, kRope>), grid, block,
                         0, stream, a, a.block_tables, a.context_lens, a.slot_mapping,
                         a.positions);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL((decode_mfma_sk_kernel<64, HPW, NBUF, MINW, KT, OT, false>), grid, block,
                         0, stream, a, a.block_tables, a.context_lens, a.slot_mapping,
                         a.positions);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  });
}

}  // namespace pagedkv
