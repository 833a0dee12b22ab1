// Multi-query causal attention over the paged cache: prefill, chunked prefill and recompute.
//
// Sequence b contributes Q_b query rows, its last Q_b logical positions; query i sits at
// position p = L_b - Q_b + i and attends to positions 0..p through the block table. This is
// the causal attention the Llama engine runs for prefill and recomputation ("vLLM-Style Llama
// Inference Engine with Tensor Parallelism", Features and scope / Implemented; How it works,
// step 4), done over the paged cache as the ragged, padding-free attention over block tables
// that llm-stack's Roadmap plans, with grouped-query heads.
//
// Work decomposition: a workgroup of 4 waves takes one KV head g of one sequence and
// 4*NB*R consecutive query tokens; each wave owns NB MFMA N blocks of 16 query rows, each
// block R = 16/G tokens x the G query heads of g. Query tiles are counted from the end of each
// sequence and the tile index is the slowest grid dimension, so every sequence's last tile
// (the most keys under the causal mask) is dispatched first: a longest-job-first order for the
// uneven causal work.
//
// Key split: when a batch has too few query tiles to fill the device and some contexts are
// long (a short chunk appended to a long cached prefix), one tile's keys would be a long serial
// chain for a few workgroups. The keys are then cut into partitions of part_keys and each
// (tile, partition) is a workgroup of its own, which leaves each row's partial (unnormalised
// output, reference max, sum) for the partition merge of the decode path, with the query
// tokens in place of the batch. A partition past a tile's keys marks its rows as empty; a
// tile whose keys fit in one partition is written out directly and its rows marked done, so
// the merge (in the form that skips done rows and empty partitions) does not touch them.
//
// The four waves read the same keys. Each 32-key pair (both 16-token blocks, K and V) is
// brought from memory once per workgroup: every thread loads 16-byte pieces into registers,
// which are written to one of two LDS buffers while the waves compute on the other; one
// barrier per pair. Each wave then takes its MFMA operands from LDS (K rows as they are, V^T
// through gfx950's transposing LDS read) and runs the tiles of mfma_tiles.h on its NB blocks,
// with a per-lane causal mask on the pairs that reach past its first row. Key slots at or past the
// workgroup's last position are stored as zeros, so stale cache contents (NaN included) never
// reach p.V; every such key is after every row's position, so the causal mask gives it
// weight 0. Rows are written normalised.
#include "launch.h"
#include "mfma_tiles.h"

#include <mutex>

namespace pagedkv {

namespace {

constexpr int kPairRows = 32;  // keys per staged pair

// LDS row pitch in bytes: a token row of D 16-bit values plus 32 bytes. The pad staggers the
// rows one wave reads together across the banks; 32 bytes measured half the bank conflicts of
// 16 or 48 (and no more than 64 or 96), no pad four times as many.
#ifndef PAGEDKV_LDS_PAD
#define PAGEDKV_LDS_PAD 32
#endif
template <int D> constexpr int lds_pitch() { return D * 2 + PAGEDKV_LDS_PAD; }

template <int D> struct LdsPair {
  alignas(16) unsigned char k[kPairRows * lds_pitch<D>()];
  alignas(16) unsigned char v[kPairRows * lds_pitch<D>()];
};

// One thread's share of a pair, kPieces 16-byte pieces of K and of V. Piece x of thread t is
// row r = (t + 256x) / (D/8) of the pair (rows 0-15: first block, 16-31: second) and 16 bytes
// at column (t + 256x) % (D/8). With 64 threads covering 64/(D/8) whole rows, the block a
// piece falls in is the same for the whole wave, so block base addresses stay scalar and a
// load is a scalar base plus a per-thread 32-bit offset fixed for the whole kernel.
// The kernel reads the pools as 16-token blocks. A cache block of 16 << sh tokens holds the
// same memory as 16-token blocks p << sh .. (p << sh) + (1 << sh) - 1, so 16-token block j of
// a sequence is that block of table entry j >> sh (sh = 0 for 16-token blocks: the plain
// table entry, at the cost of two scalar operations and no branch). -1 when the entry is
// outside the pool.
__device__ __forceinline__ int sub_block_id(const int32_t* table, int j, int sh,
                                           int64_t num_blocks) {
  const int p = table[j >> sh];
  return p >= 0 && (int64_t)p < num_blocks ? (p << sh) | (j & ((1 << sh) - 1)) : -1;
}

template <int D> struct Stager {
  static constexpr int kCPR = D / 8;                           // pieces per row
  static constexpr int kPieces = kPairRows * kCPR / 256;      // per thread: D 64 -> 1, 128 -> 2
  uint32_t goff[kPieces];  // byte offset of the piece inside its block (row, head, column)
  uint32_t loff[kPieces];  // byte offset of the piece in an LdsPair buffer
  int row[kPieces];        // r
  int blk[kPieces];        // 0 or 1: block of the pair (uniform over the wave)

  // One staged pair in flight: the thread's pieces and the pair's edge state.
  struct Regs {
    uint4 k[kPieces], v[kPieces];
    int zero_a, zero_b;  // uniform: block A / B of the pair is absent or invalid
    int tail_from;       // rows r >= tail_from of the pair are zero (32: none)
  };

  __device__ __forceinline__ void init(int wave, size_t row_stride, size_t head_off) {
#pragma unroll
    for (int x = 0; x < kPieces; ++x) {
      const int idx = threadIdx.x + 256 * x;
      const int r = idx / kCPR, c = idx % kCPR;
      row[x] = r;
      blk[x] = (wave * (64 / kCPR) + x * (256 / kCPR)) / 16;
      goff[x] = (uint32_t)(((size_t)(r & 15) * row_stride + head_off + 8 * c) * 2);
      loff[x] = (uint32_t)(r * lds_pitch<D>() + 16 * c);
    }
  }

  // Load pair `pair` into r. The loads are only issued here; the data is first used by
  // commit(), after the current pair's compute, so their latency hides behind it. A block id outside
  // the pool reads block 0 instead, and such a block, and rows at or past tok1 (only in the
  // last pair), are stored as zeros by commit().
  __device__ __forceinline__ void load(Regs& rg, const PrefillArgs& a, const int32_t* table,
                                       int nblk, int tok1, size_t row_stride, int pair) const {
    const int jA = 2 * pair;
    const int sh = __builtin_ctz((unsigned)a.block_size) - 4;  // block_size = 16 << sh
    const int idA = sub_block_id(table, jA, sh, a.num_blocks);
    const int idB = jA + 1 < nblk ? sub_block_id(table, jA + 1, sh, a.num_blocks) : -1;
    const bool okA = idA >= 0;
    const bool okB = idB >= 0;
    rg.zero_a = !okA;
    rg.zero_b = !okB;
    rg.tail_from = min(tok1 - 32 * pair, 32);
    const size_t bbytes = (size_t)16 * row_stride * 2;  // bytes of one block
    const char* kc = reinterpret_cast<const char*>(a.k_cache);
    const char* vc = reinterpret_cast<const char*>(a.v_cache);
    const int safe_a = okA ? idA : 0, safe_b = okB ? idB : 0;
#pragma unroll
    for (int x = 0; x < kPieces; ++x) {
      // The block is the same for the whole wave; its id taken from the first lane stays in a
      // scalar register (a per-lane select of it cost more vector instructions per pair).
      const int id = __builtin_amdgcn_readfirstlane(blk[x] ? safe_b : safe_a);
      rg.k[x] = *reinterpret_cast<const uint4*>(kc + (size_t)id * bbytes + goff[x]);
      rg.v[x] = *reinterpret_cast<const uint4*>(vc + (size_t)id * bbytes + goff[x]);
    }
  }

  __device__ __forceinline__ void commit(Regs& rg, LdsPair<D>& p) const {
    if (rg.zero_a || rg.zero_b || rg.tail_from < 32) {  // uniform: only an edge pair
#pragma unroll
      for (int x = 0; x < kPieces; ++x) {
        const bool ok = !(blk[x] ? rg.zero_b : rg.zero_a) && row[x] < rg.tail_from;
        rg.k[x] = select4(ok, rg.k[x], make_uint4(0, 0, 0, 0));
        rg.v[x] = select4(ok, rg.v[x], make_uint4(0, 0, 0, 0));
      }
    }
#pragma unroll
    for (int x = 0; x < kPieces; ++x) {
      *reinterpret_cast<uint4*>(p.k + loff[x]) = rg.k[x];
      *reinterpret_cast<uint4*>(p.v + loff[x]) = rg.v[x];
    }
  }
};

// 4 x 16-bit elements of LDS through the transposing read ds_read_b64_tr_b16. Within each
// group of 16 lanes, lane i receives element i % 4 of the 8 bytes that lanes 4j + i / 4
// address, for j = 0..3.
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(__attribute__((address_space(3))) const unsigned char*)p);
  return __builtin_bit_cast(uint2, r);
}

// A wave's MFMA operands of a staged pair:
//   ka / kb: K rows n16 (first block) and 16 + n16 (second), columns 32ch + 8kg .. +7;
//   vt[e]:   V^T of output columns 16e .. 16e+15: lane (n16, kg) holds column 16e + n16 of the
//            keys in its slots 8kg .. 8kg+7, i.e. rows 4kg .. 4kg+3 of the first block and of
//            the second. Each half is one transposing read in which lane (n16, kg) addresses
//            row 4kg + n16/4 (of the block) at column 16e + 4*(n16 % 4).
template <int D, int NCH, int EPL>
__device__ __forceinline__ void read_pair(uint4 (&ka)[NCH], uint4 (&kb)[NCH], uint4 (&vt)[EPL],
                                          const LdsPair<D>& p, int n16, int kg) {
  constexpr int P = lds_pitch<D>();
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    ka[ch] = *reinterpret_cast<const uint4*>(p.k + n16 * P + 2 * (32 * ch + 8 * kg));
    kb[ch] = *reinterpret_cast<const uint4*>(p.k + (16 + n16) * P + 2 * (32 * ch + 8 * kg));
  }
  const unsigned char* va = p.v + (4 * kg + n16 / 4) * P + 8 * (n16 % 4);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const uint2 lo = lds_read_tr16(va + 32 * e);
    const uint2 hi = lds_read_tr16(va + 16 * P + 32 * e);
    vt[e] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

}  // namespace

// Maxima of scores without the canonicalising v_max x, x that IEEE mode puts in front of fmaxf
// on values the compiler cannot prove quiet (the masked scores and the cross-lane exchanges
// here): no operand is a signalling NaN, and only the rescale decision reads the result.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8_raw(const float (&x)[8]) {
  return max3_raw(max3_raw(x[0], x[1], x[2]), max3_raw(x[3], x[4], x[5]),
                  max3_raw(x[6], x[7], x[7]));
}
// The maximum over the 4 lanes n16 + 16 kg of a row (the cross-lane exchange of row4_max).
__device__ __forceinline__ float row4_max_raw(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = max3_raw(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return max3_raw(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

// Several N blocks of 16 query rows against one pair of key blocks, from operands already in
// registers: the K rows of both blocks as the A operand of q.K, and vt[e], the V^T operand of
// output-column group e. Every (pair, block) shares them, so one pass over the keys feeds
// 16*NB rows. Block nb's rows sit at positions row_pos[nb] (per lane); keys after a row's
// position get weight 0 when `active` (uniform) says some key of the pair lies after the
// earliest row. No key of the pair is stale (the caller zeroes those and the causal mask
// covers them).
//
// The online-softmax update is the decode one (softmax_step), regrouped over the blocks: every
// block's q.K^T first, then the maxima, then one rescaling branch for all blocks (a block whose
// maximum did not move multiplies by exactly 1, so the results are those of one update per
// block), then each block's weights and P.V. With no branch between one block's products and
// the next block's exponentials, the compiler can issue the vector work of block nb + 1 while
// the matrix products of block nb run. (Scaling inside the exponent's fused multiply-add,
// 2^(raw * scale_log2 - m), saves one instruction per score but loses the exact weight 1 of a
// row's largest score, and with it the exact value row of a row that sees one key.)
template <int KT, int NCH, int EPL, int NB>
__device__ __forceinline__ void pair_compute_rows(const uint4 (&ka)[NCH], const uint4 (&kb)[NCH],
                                                  const uint4 (&vt)[EPL],
                                                  WaveState<EPL> (&st)[NB],
                                                  const uint4 (&qb)[NB][NCH], float sl2, int kg,
                                                  const int (&row_pos)[NB], int key0,
                                                  bool active) {
  constexpr int BS = 16;
  floatx4 sA[NB], sB[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    sA[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    sB[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      sA[nb] = mfma16x16x32<KT>(ka[ch], qb[nb][ch], sA[nb]);
      sB[nb] = mfma16x16x32<KT>(kb[ch], qb[nb][ch], sB[nb]);
    }
  }
  float s[NB][8];  // scores in log2 units; -inf past a row's position
  float mn[NB];
  bool upd[NB];
  bool any_upd = false;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[nb][i] = sA[nb][i] * sl2;
      s[nb][4 + i] = sB[nb][i] * sl2;
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[nb][i] = key0 + 4 * kg + i <= row_pos[nb] ? s[nb][i] : kNegInf;
        s[nb][4 + i] = key0 + BS + 4 * kg + i <= row_pos[nb] ? s[nb][4 + i] : kNegInf;
      }
    }
    const float mx = row4_max_raw(max8_raw(s[nb]));
    mn[nb] = max3_raw(st[nb].m_run, mx, mx);
    upd[nb] = mn[nb] > st[nb].m_run + kRescaleSlack;  // also true while m_run is -inf
    any_upd = any_upd || upd[nb];
  }
  if (__any(any_upd)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float m_new = upd[nb] ? mn[nb] : st[nb].m_run;
      const float alpha =
          upd[nb] ? fast_exp2(st[nb].m_run - (m_new == kNegInf ? 0.f : m_new)) : 1.f;
      st[nb].l_run *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) st[nb].acc[e] *= alpha;
      st[nb].m_run = m_new;
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float mu = (st[nb].m_run == kNegInf ? 0.f : st[nb].m_run) - kWeightLift<KT>;
    float pw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pw[i] = fast_exp2(s[nb][i] - mu);
    float psum = pw[0];  // the same bits as 0 + pw[0] (weights are >= 0), one add fewer
#pragma unroll
    for (int i = 1; i < 8; ++i) psum += pw[i];
    st[nb].l_run += psum;
    uint4 phi, plo;
    split_weights<KT>(pw, phi, plo);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      st[nb].acc[e] = mfma16x16x32<KT>(vt[e], phi, st[nb].acc[e]);
      st[nb].acc[e] = mfma16x16x32<KT>(vt[e], plo, st[nb].acc[e]);
    }
  }
}

template <int D, int NW, int NB, int MINW, int KT, int OT>
__global__ void __launch_bounds__(NW * 64, MINW)
prefill_mfma_kernel(const PrefillArgs a) {
  constexpr int NCH = D / 32;
  constexpr int EPL = D / 16;
  static_assert(NW == 4, "the staging split assumes 256 threads");
  __shared__ LdsPair<D> buf[2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int kg = lane >> 4;

  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int R = 16 / G;  // query tokens per N block
  // Tiles counted from the end of each sequence, tile index slowest (see the top of the file),
  // then the key partition, then (sequence, KV head).
  const int unit = blockIdx.x;
  const int nbg = a.batch * Hkv;
  const int bg = unit % nbg;
  const int part = (unit / nbg) % a.nparts;
  const int tile = unit / (nbg * a.nparts);
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int q0 = a.cu_seqlens_q[b];
  int Q = a.cu_seqlens_q[b + 1] - q0;
  Q = Q < 0 ? 0 : Q;
  const int wg_end = Q - tile * NW * NB * R;  // one past the workgroup's last token
  if (wg_end <= 0) return;                    // uniform over the workgroup: before any barrier
  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * a.block_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);

  // This wave's tokens (possibly none: it still loads and meets every barrier).
  const int tok_end = wg_end - wave * NB * R;
  const int tok_base = tok_end - NB * R;
  const bool wave_rows = tok_end > 0;
  const int head = n16 % G;
  int tok[NB], row_pos[NB];
  bool row_ok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    tok[nb] = tok_base + nb * R + n16 / G;
    row_ok[nb] = n16 < R * G && tok[nb] >= 0;
    row_pos[nb] = row_ok[nb] ? L - Q + tok[nb] : -1;
  }
  const int first_tok = tok_base > 0 ? tok_base : 0;
  const int p_min = L - Q + first_tok;
  const int p_max = L - Q + tok_end - 1;        // this wave's last position
  const int wg_p_max = L - Q + wg_end - 1;      // the workgroup's (wave 0's) last position
  const int tok1 = wg_p_max + 1 > 0 ? wg_p_max + 1 : 0;
  const int nblk = (tok1 + 15) / 16;
  const int np = (nblk + 1) / 2;
  // Key split: this workgroup takes pairs [pair_lo, pair_hi) of the tile's np pairs.
  const int pair_lo = part * (a.part_keys / kPairRows);
  const int pair_hi = min(pair_lo + a.part_keys / kPairRows, np);

  uint4 qb[NB][NCH];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint16_t* qrow =
        a.q + ((size_t)(q0 + (row_ok[nb] ? tok[nb] : first_tok)) * Hq + (size_t)g * G + head) * D +
        8 * kg;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qb[nb][c] = make_uint4(0, 0, 0, 0);
      if (row_ok[nb]) qb[nb][c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
    }
  }

  WaveState<EPL> st[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    st[nb].m_run = kNegInf;
    st[nb].l_run = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st[nb].acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const size_t row_stride = (size_t)Hkv * D;
  const size_t head_off = (size_t)g * D;
  const float sl2 = a.scale_log2;
  const int nparts = a.nparts;
  // With a key split, a tile whose keys fit in one partition is not split: partition 0 writes
  // its rows out directly and marks them done for the merge, the other partitions have nothing
  // to do. A split tile's partitions past its keys mark their rows as having no keys, so the
  // merge never reads their partial outputs. (Uniform over the workgroup, before any barrier.)
  const bool tile_split = nparts > 1 && np > a.part_keys / kPairRows;
  if (nparts > 1 && !tile_split && part != 0) return;
  if (tile_split && pair_lo >= np) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (row_ok[nb] && kg == 0) {
        const size_t pr = ((size_t)(q0 + tok[nb]) * Hq + (size_t)g * G + head) * nparts + part;
        a.ws_ml[pr * 2 + 0] = kNegInf;
        a.ws_ml[pr * 2 + 1] = 0.f;
      }
    return;
  }

  if (pair_lo < pair_hi) {
    // Two register sets, the loop unrolled by two: pair k + 2's loads are issued while pair
    // k is computed from LDS and pair k + 1 waits in the other set. (The compiler's wait
    // counting, merging the paths around the conditional loads and commits, still waits for
    // both sets at each commit, so mostly one pair is in flight; unconditional loads and
    // commits fixed the commit waits but not the loop head's, and measured the same.)
    Stager<D> s;
    typename Stager<D>::Regs r0, r1;
    s.init(wave, row_stride, head_off);
    s.load(r0, a, table, nblk, tok1, row_stride, pair_lo);
    if (pair_lo + 1 < pair_hi) s.load(r1, a, table, nblk, tok1, row_stride, pair_lo + 1);
    s.commit(r0, buf[0]);
    __syncthreads();
    auto step = [&](int k, typename Stager<D>::Regs& next, typename Stager<D>::Regs& spare) {
      const int cur = (k - pair_lo) & 1;
      if (k + 2 < pair_hi) s.load(spare, a, table, nblk, tok1, row_stride, k + 2);  // uniform
      const int key0 = 32 * k;
      if (wave_rows && key0 <= p_max) {
        uint4 ka[NCH], kb[NCH], vt[EPL];
        read_pair<D>(ka, kb, vt, buf[cur], n16, kg);
        pair_compute_rows<KT>(ka, kb, vt, st, qb, sl2, kg, row_pos, key0, key0 + 31 > p_min);
      }
      if (k + 1 < pair_hi) s.commit(next, buf[cur ^ 1]);
      __syncthreads();
    };
    for (int k = pair_lo; k < pair_hi; k += 2) {
      step(k, r1, r0);
      if (k + 1 < pair_hi) step(k + 1, r0, r1);
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l_run = st[nb].l_run;
    l_run = row4_sum(l_run);
    if (!row_ok[nb]) continue;
    const size_t row = (size_t)(q0 + tok[nb]) * Hq + (size_t)g * G + head;
    if (!tile_split) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      const size_t o = row * D;
      // acc[e][i] is output column 16e + 4kg + i
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        store_out4<OT>(a.out, o + 16 * e + 4 * kg, st[nb].acc[e][0] * inv,
                       st[nb].acc[e][1] * inv, st[nb].acc[e][2] * inv,
                       st[nb].acc[e][3] * inv);
      if (nparts > 1 && kg == 0) {  // done: the merge leaves this row alone
        a.ws_ml[row * nparts * 2 + 0] = kNegInf;
        a.ws_ml[row * nparts * 2 + 1] = -1.f;
      }
    } else {
      // This partition's partial for the merge: unnormalised output, reference max and sum
      // (a row whose position lies before the partition saw no keys: -inf and 0).
      const size_t pr = row * nparts + part;
      float* o = a.ws_acc + pr * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        *reinterpret_cast<float4*>(o + 16 * e + 4 * kg) =
            make_float4(st[nb].acc[e][0], st[nb].acc[e][1], st[nb].acc[e][2], st[nb].acc[e][3]);
      if (kg == 0) {
        a.ws_ml[pr * 2 + 0] = st[nb].m_run;
        a.ws_ml[pr * 2 + 1] = l_run;
      }
    }
  }
}

bool supported_prefill(int head_dim, int group, int block_size) {
  // 16-token blocks or larger powers of two up to 1024 (the loader shifts block indices)
  return block_size >= 16 && block_size <= 1024 && (block_size & (block_size - 1)) == 0 &&
         (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

int prefill_tokens_per_group(int group, int nb) { return kWavesPerGroup * nb * (16 / group); }

template <int NB> constexpr int prefill_min_waves() { return NB == 4 ? 1 : 2; }

// Register use (and so occupancy) is taken from the bf16 -> fp32 instance of each (D, NB);
// the other formats differ only in conversions and the output store.
template <int D, int NB>
static const void* prefill_kernel_ptr() {
  return reinterpret_cast<const void*>(
      &prefill_mfma_kernel<D, kWavesPerGroup, NB, prefill_min_waves<NB>(), kDtBf16, kDtF32>);
}

// Workgroups of the (D, NB) variant one CU holds at once, asked of the runtime once per
// device (it follows from the variant's registers and LDS).
static int prefill_groups_per_cu(int head_dim, int nb_index) {
  static std::mutex mu;
  static int cache[256][2][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 1;
  const int di = head_dim == 128 ? 1 : 0;
  std::lock_guard<std::mutex> lock(mu);
  int& slot = cache[dev][di][nb_index];
  if (slot == 0) {
    static const void* const ptrs[2][3] = {
        {prefill_kernel_ptr<64, 1>(), prefill_kernel_ptr<64, 2>(), prefill_kernel_ptr<64, 4>()},
        {prefill_kernel_ptr<128, 1>(), prefill_kernel_ptr<128, 2>(), prefill_kernel_ptr<128, 4>()}};
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ptrs[di][nb_index], kWavesPerGroup * 64,
                                                     0) != hipSuccess)
      n = 1;
    slot = n > 0 ? n : 1;
  }
  return slot;
}

// N blocks of 16 query rows per wave. A larger NB computes more rows per staged pair but holds
// more registers, and it cuts the query rows into fewer workgroups. The launch takes NB = 2
// when its workgroups (counted from the total query rows, a lower bound for ragged batches)
// fill the resident slots at least once, and NB = 1 otherwise (a 2 x 2048-token recompute at
// head_dim 64, 1024 workgroups for 768 slots, measured 4% faster with NB = 2). NB = 4 (callers may ask for it) needs more registers than a SIMD holds
// for two waves and measured slower on every workload. A build may pin NB with
// PAGEDKV_PREFILL_NB.
int prefill_rows_per_wave(int64_t num_tokens, int num_kv_heads, int head_dim, int group,
                          int cus) {
#ifdef PAGEDKV_PREFILL_NB
  (void)num_tokens; (void)num_kv_heads; (void)head_dim; (void)group; (void)cus;
  return PAGEDKV_PREFILL_NB;
#else
  const int64_t per_group = prefill_tokens_per_group(group, 2);
  const int64_t units = (int64_t)num_kv_heads * ((num_tokens + per_group - 1) / per_group);
  const int64_t slots = (int64_t)cus * prefill_groups_per_cu(head_dim, 1);
  return units >= slots ? 2 : 1;
#endif
}

template <int D, int KT, int OT>
static hipError_t launch_prefill_d(const PrefillArgs& a, unsigned grid, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  switch (a.nb) {
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 1, prefill_min_waves<1>(), KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 2, prefill_min_waves<2>(), KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 4, prefill_min_waves<4>(), KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  const unsigned units =
      (unsigned)((long long)a.batch * a.num_kv_heads * a.ntiles * a.nparts);
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    if (a.head_dim == 128) return launch_prefill_d<128, KT, OT>(a, units, stream);
    if (a.head_dim == 64) return launch_prefill_d<64, KT, OT>(a, units, stream);
    return hipErrorInvalidValue;
  });
}

}  // namespace pagedkv
