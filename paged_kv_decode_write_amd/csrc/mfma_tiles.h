// Register tiles shared by the matrix-core attention kernels (decode and multi-query causal):
// one wave streams pairs of 16-token blocks of one KV head and runs, per pair,
//   S^T = K_tile . Q^T   (v_mfma_f32_16x16x32_bf16 or _f16 for fp16 inputs: M = 16 keys,
//                        N = 16 query rows, K = 32 columns of D; K rows feed the A operand
//                        from global memory),
//   online softmax per query row (lazily rescaled reference max, shared by the 4 lanes of
//   a row), and
//   O^T += V^T . P^T     (M = 16 output columns, N = 16 rows, K = 32 keys; keys contracted in
//                        the order the scores already sit in the lanes, V^T transposed in
//                        registers with v_perm_b32, p split into a hi + lo pair in the
//                        input format).
// Lane (n16 = lane % 16, kg = lane / 16) owns query row n16; it holds scores of keys
// 4kg..4kg+3 of each block of the pair and output columns EPL*(4kg+i)+e of its row.
#pragma once

#include "device_common.h"

namespace pagedkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));  // v_cvt_pkrtz result
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One 16x16x32 product with fp32 accumulate; a and b hold 8 packed 16-bit values of the input
// format KT (bf16 or fp16).
template <int KT>
__device__ __forceinline__ floatx4 mfma16x16x32(const uint4& a, const uint4& b,
                                                const floatx4& c) {
  if constexpr (KT == kDtF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// c ? a : b for 16-byte values, component by component (a select of the whole struct would
// go through memory).
__device__ __forceinline__ uint4 select4(bool c, const uint4& a, const uint4& b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// Low / high bf16 halves of two words packed into one word (x's half first).
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Loads with the non-temporal hint (global_load ... nt): the data is streamed once, and the
// lines are not kept for reuse. Used for V rows, which a wave reads as whole cache lines (16
// lanes x 16 or 8 bytes of one row). Measured on cold decode: 64 x 8192 tokens 358 -> 322 us,
// 2 x 32768 49.5 -> 45.4 us, the ragged 48-sequence batch 96 -> 92 us. K rows are read as
// 64-byte halves of a line by two instructions (the MFMA operand layout), and with the hint
// on them the second half was fetched again: more HBM bytes and slower, so K loads stay plain.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt16(const uint16_t* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_nt8(const uint16_t* p) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

// Row of EPL consecutive 16-bit values (EPL = 8: 16 bytes, EPL = 4: 8 bytes), loaded with the
// non-temporal hint.
template <int EPL> struct VRow;
template <> struct VRow<8> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = load_nt16(p); }
  __device__ __forceinline__ void keep_if(bool v) {
    w.x = v ? w.x : 0u; w.y = v ? w.y : 0u; w.z = v ? w.z : 0u; w.w = v ? w.w : 0u;
  }
  __device__ __forceinline__ void take_if(bool c, const VRow& o) {
    w.x = c ? o.w.x : w.x; w.y = c ? o.w.y : w.y; w.z = c ? o.w.z : w.z; w.w = c ? o.w.w : w.w;
  }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = w; }
  __device__ __forceinline__ uint32_t word(int i) const {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
  }
};
template <> struct VRow<4> {
  uint2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = load_nt8(p); }
  __device__ __forceinline__ void keep_if(bool v) { w.x = v ? w.x : 0u; w.y = v ? w.y : 0u; }
  __device__ __forceinline__ void take_if(bool c, const VRow& o) {
    w.x = c ? o.w.x : w.x; w.y = c ? o.w.y : w.y;
  }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint2*>(p) = w; }
  __device__ __forceinline__ uint32_t word(int i) const { return i == 0 ? w.x : w.y; }
};

// Slack of the lazily updated softmax reference max, in log2 units (weights <= 2^8).
constexpr float kRescaleSlack = 8.f;

// Exponent lift (log2) of the weights that enter p.V. bf16 has fp32's exponent range and
// needs none. fp16 stops at 2^-24: weights are taken as 2^(s - m + 7) (largest 2^15, below
// the fp16 maximum 65504), so a weight still counts down to 2^-31 of the reference. The sum
// carries the same factor, so it cancels in acc / l and in the partition merge.
template <int KT> constexpr float kWeightLift = KT == kDtF16 ? 7.f : 0.f;

// Two weights a, b (neighbouring token slots of the P^T operand) as hi + lo in the input
// format, with p = hi + lo + O(2^-16 p). bf16: hi is p rounded to nearest even, two per v_cvt_pk; the
// remainders p - hi come from v_dot2c_f32_bf16 against (-1, 0) and (0, -1), one instruction
// each (p - hi is exact in fp32, and the other product is 0), and lo is them rounded. fp16: hi
// is p rounded toward zero (v_cvt_pkrtz_f16_f32), the remainders likewise from
// v_dot2_f32_f16, and lo is them rounded toward zero.
template <int KT>
__device__ __forceinline__ void split_weight_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  if constexpr (KT == kDtF16) {
    // (-1, 0) and (0, -1) as packed fp16, in scalar registers as for bf16 below
    uint32_t neg_first = 0x0000bc00u, neg_second = 0xbc000000u;
    asm("" : "+s"(neg_first));
    asm("" : "+s"(neg_second));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(a, b);
    const h2 hh = __builtin_bit_cast(h2, h);
    const fp16x2 l = __builtin_amdgcn_cvt_pkrtz(
        __builtin_amdgcn_fdot2(hh, __builtin_bit_cast(h2, neg_first), a, false),
        __builtin_amdgcn_fdot2(hh, __builtin_bit_cast(h2, neg_second), b, false));
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  } else {
    // (-1, 0) and (0, -1) as packed bf16, held in scalar registers: written as constants, the
    // first one became the inline constant -1.0, which the instruction reads as (0, -1).
    uint32_t neg_first = 0x0000bf80u, neg_second = 0xbf800000u;
    asm("" : "+s"(neg_first));
    asm("" : "+s"(neg_second));
    const floatx2 v = {a, b};
    const bf16x2 h = __builtin_convertvector(v, bf16x2);
    const floatx2 r = {
        __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg_first), a, false),
        __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg_second), b, false)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
  }
}

// All eight weights p[0..7] of a lane, as the hi and lo P^T operands.
template <int KT>
__device__ __forceinline__ void split_weights(const float (&p)[8], uint4& hi, uint4& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_weight_pair<KT>(p[2 * q], p[2 * q + 1], hw[q], lw[q]);
  hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

// Per-lane softmax state of one wave: the head is n16 = lane % 16; lanes of the same head
// (kg = 0..3) share m_run and hold disjoint output columns.
template <int EPL> struct WaveState {
  floatx4 acc[EPL];  // O^T: acc[e][i] = out[head n16][EPL*(4kg+i) + e] (unnormalised)
  float m_run;       // reference max (log2 units)
  float l_run;       // this lane's share of the running sum
};

// Registers of one block pair in flight: K rows as the A operand of q.K, V rows as loaded.
template <int NCH, int EPL> struct PairTile {
  uint4 ka[NCH], kb[NCH];
  VRow<EPL> vr[8];
  int lastA, lastB;  // valid rows in each block (0: block absent or invalid)
  int tA;            // position of the first row of the pair
};

// Marks the loads of a tile as used by `tie`, a value the caller then stores. A kernel that
// issues loads before a branch that may exit passes the value it stores on the exit path: a
// load whose value is used on both sides of the branch cannot be moved below it, so it stays
// ahead of the wait the branch needs, and only the exit path waits for it. The asm is empty
// (tie keeps its value) and not volatile, so the compiler sees no memory access in it; one
// word of each load is enough, since a load is a single instruction.
__device__ __forceinline__ void keep_issued(uint32_t w, float& tie) {
  asm("" : "+v"(tie) : "v"(w));
}
template <int NCH, int EPL>
__device__ __forceinline__ void keep_issued(const PairTile<NCH, EPL>& t, float& tie) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    keep_issued(t.ka[c].x, tie);
    keep_issued(t.kb[c].x, tie);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) keep_issued(t.vr[j].word(0), tie);
}

// Fused decode step: one lane's pieces of the step's new K and V rows of its head (K columns
// 32ch + 8kg .. +7, V columns EPL*n16 .. +EPL-1), loaded once before the key loop.
template <int NCH, int EPL> struct NewRow {
  uint4 k[NCH];
  VRow<EPL> v;
};

template <int NCH, int EPL>
__device__ __forceinline__ void keep_issued(const NewRow<NCH, EPL>& r, float& tie) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) keep_issued(r.k[c].x, tie);
  keep_issued(r.v.word(0), tie);
}

template <int NCH, int EPL>
__device__ __forceinline__ void load_new_row(NewRow<NCH, EPL>& r, const uint16_t* k_row,
                                             const uint16_t* v_row, int n16, int kg) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    r.k[ch] = *reinterpret_cast<const uint4*>(k_row + 8 * kg + 32 * ch);
  r.v.load(v_row + EPL * n16);
}

// 16-bit element t (0..7) of an 8-element piece, and its replacement.
__device__ __forceinline__ uint32_t piece_word(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t piece_elem(const uint4& v, int t) {
  return (piece_word(v, t / 2) >> (16 * (t % 2))) & 0xffffu;
}
__device__ __forceinline__ void piece_set(uint4& v, int t, uint32_t h) {
  const uint32_t keep = t % 2 ? 0x0000ffffu : 0xffff0000u;
  const uint32_t put = t % 2 ? h << 16 : h;
  switch (t / 2) {
    case 0: v.x = (v.x & keep) | put; break;
    case 1: v.y = (v.y & keep) | put; break;
    case 2: v.z = (v.z & keep) | put; break;
    default: v.w = (v.w & keep) | put; break;
  }
}

template <int KT> __device__ __forceinline__ float elem_to_f32(uint32_t h) {
  return in_lo<KT>(h);
}
template <int KT> __device__ __forceinline__ uint32_t f32_to_elem(float f) {
  if constexpr (KT == kDtF16) return f32_to_f16_rne(f);
  else return f32_to_bf16_rne(f);
}

// Rotary embedding, in registers, of one lane's pieces of a query row and of a key row: the
// lane holds columns 32c + 8kg .. +7 of each (c < NCH). Pair i turns by pos * inv_freq[i]
// (fp32 product, then sincosf, then rope_rotate, then rounding to the 16-bit format, as the
// standalone RoPE kernel does). A wave needs only D/2 = 16 NCH angles, so lane l evaluates the
// sine and cosine of pair l mod D/2 once and the lanes fetch the ones they need from each
// other (ds_bpermute moves bits, so the values are those of the standalone kernel). Half
// pairing (i, i + D/2) pairs chunk c with chunk c + NCH/2 at the same offset (pair
// 32c + 8kg + t); interleaved pairing (2i, 2i+1) pairs neighbours inside a piece (pair
// 16c + 4kg + u).
template <int KT, int NCH>
__device__ __forceinline__ void rope_pieces(uint4 (&q)[NCH], uint4 (&k)[NCH], float pos,
                                            const float* inv_freq, bool interleaved, int kg,
                                            int lane) {
  constexpr int kPairs = 16 * NCH;  // D/2: 64 or 32, never more than a wave
  float sn_own, cs_own;
  sincosf(pos * inv_freq[lane % kPairs], &sn_own, &cs_own);
  const auto turn = [&](uint4& a, int ta, uint4& b, int tb, int pair) {
    const float sn = __shfl(sn_own, pair), cs = __shfl(cs_own, pair);
    float y0, y1;
    rope_rotate(elem_to_f32<KT>(piece_elem(a, ta)), elem_to_f32<KT>(piece_elem(b, tb)), cs, sn,
                y0, y1);
    piece_set(a, ta, f32_to_elem<KT>(y0));
    piece_set(b, tb, f32_to_elem<KT>(y1));
  };
  if (!interleaved) {
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int pair = 32 * c + 8 * kg + t;
        turn(q[c], t, q[c + NCH / 2], t, pair);
        turn(k[c], t, k[c + NCH / 2], t, pair);
      }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pair = 16 * c + 4 * kg + u;
        turn(q[c], 2 * u, q[c], 2 * u + 1, pair);
        turn(k[c], 2 * u, k[c], 2 * u + 1, pair);
      }
  }
}

// Put the new row in place of position sub_pos (-1: none) of a loaded pair, by selects on data
// that has already arrived: the cache slot of that position is being written by the same
// launch, so what its load returned is discarded.
template <int NCH, int EPL>
__device__ __forceinline__ void use_new_row(PairTile<NCH, EPL>& t, const NewRow<NCH, EPL>& r,
                                            int sub_pos, int n16, int kg) {
  constexpr int BS = 16;
  const int rel = sub_pos - t.tA;  // the new token's row in the pair, if 0 <= rel < 32
  if (rel >= 0 && rel < 2 * BS) {  // uniform
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      t.ka[ch] = select4(rel == n16, r.k[ch], t.ka[ch]);
      t.kb[ch] = select4(rel == BS + n16, r.k[ch], t.kb[ch]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) t.vr[j].take_if(rel == (j / 4) * BS + 4 * kg + (j % 4), r.v);
  }
}

template <int D> struct PairCtx {
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* table;  // this sequence's block-table row
  size_t row_stride;     // elements between token rows (Hkv * D)
  size_t head_off;       // g * D
  int64_t num_blocks;
  int blk0, blk1, tok1, wave, n16, kg;
};

// Block ids of this wave's pair k (uniform, scalar loads).
template <int D, int NW>
__device__ __forceinline__ int2 pair_ids(const PairCtx<D>& c, int k) {
  const int jA = c.blk0 + 2 * (c.wave + NW * k);
  const int pA = c.table[jA];
  const int pB = jA + 1 < c.blk1 ? c.table[jA + 1] : -1;
  return make_int2(pA, pB);
}

// Issue the loads of the pair whose first block is block jA of the sequence. An invalid
// block id is replaced by block 0 (always in the pool); pair_valid then gives it no valid
// rows, so its contents never reach the result. Only the ids and the constant parts of the
// context are used, so a kernel may issue a pair before it knows the context length.
template <int D, int NCH, int EPL>
__device__ __forceinline__ void pair_issue(PairTile<NCH, EPL>& t, const PairCtx<D>& c, int2 ids,
                                           int jA) {
  constexpr int BS = 16;
  const bool okA = ids.x >= 0 && (int64_t)ids.x < c.num_blocks;
  const bool okB = ids.y >= 0 && (int64_t)ids.y < c.num_blocks;
  const size_t bA = (size_t)(okA ? ids.x : 0) * BS * c.row_stride + c.head_off;
  const size_t bB = (size_t)(okB ? ids.y : 0) * BS * c.row_stride + c.head_off;
  const size_t koff = (size_t)c.n16 * c.row_stride + 8 * c.kg;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    t.ka[ch] = *reinterpret_cast<const uint4*>(c.k_cache + bA + koff + 32 * ch);
    t.kb[ch] = *reinterpret_cast<const uint4*>(c.k_cache + bB + koff + 32 * ch);
  }
  const size_t voff = (size_t)(4 * c.kg) * c.row_stride + EPL * c.n16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.vr[j].load(c.v_cache + bA + voff + (size_t)j * c.row_stride);
    t.vr[4 + j].load(c.v_cache + bB + voff + (size_t)j * c.row_stride);
  }
  t.tA = jA * BS;
}

// Valid rows of each block of a pair issued with these ids (0 for an invalid id; <= 0 for a
// block at or past tok1).
template <int D, int NCH, int EPL>
__device__ __forceinline__ void pair_valid(PairTile<NCH, EPL>& t, const PairCtx<D>& c, int2 ids,
                                           int jA) {
  constexpr int BS = 16;
  const bool okA = ids.x >= 0 && (int64_t)ids.x < c.num_blocks;
  const bool okB = ids.y >= 0 && (int64_t)ids.y < c.num_blocks;
  const int tA = jA * BS;
  t.lastA = okA ? min(c.tok1 - tA, BS) : 0;
  t.lastB = okB ? min(c.tok1 - tA - BS, BS) : 0;
}

// Issue the loads of this wave's pair k (see pair_issue) and set its valid rows.
template <int D, int NW, int NCH, int EPL>
__device__ __forceinline__ void pair_load(PairTile<NCH, EPL>& t, const PairCtx<D>& c, int2 ids,
                                          int k) {
  const int jA = c.blk0 + 2 * (c.wave + NW * k);
  pair_issue(t, c, ids, jA);
  pair_valid(t, c, ids, jA);
}

// V^T operand of output column set e: 8 token slots of column EPL*n16 + e, gathered from the
// 8 loaded V rows with v_perm_b32 (a 16-bit shuffle, the same for both input formats).
template <int NCH, int EPL>
__device__ __forceinline__ uint4 vt_operand(const PairTile<NCH, EPL>& t, int e) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t x = t.vr[2 * q].word(e / 2), y = t.vr[2 * q + 1].word(e / 2);
    w[q] = (e & 1) ? pack_hi(x, y) : pack_lo(x, y);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Zero the V rows past a block's valid rows: stale slots may hold NaN bits, and 0 * NaN would
// poison p.V even where the weight is 0.
template <int NCH, int EPL>
__device__ __forceinline__ void clear_stale_rows(PairTile<NCH, EPL>& t, int kg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.vr[i].keep_if(4 * kg + i < t.lastA);
    t.vr[4 + i].keep_if(4 * kg + i < t.lastB);
  }
}

// Scores of one pair for one 16-row N block: q.K on the matrix cores, scaled to log2 units.
template <int KT, int NCH, int EPL>
__device__ __forceinline__ void pair_scores(const PairTile<NCH, EPL>& t, const uint4 (&qb)[NCH],
                                            float sl2, float (&s)[8]) {
  floatx4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    sA = mfma16x16x32<KT>(t.ka[ch], qb[ch], sA);
    sB = mfma16x16x32<KT>(t.kb[ch], qb[ch], sB);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = sA[i] * sl2;
    s[4 + i] = sB[i] * sl2;
  }
}

// Positions past a block's valid rows: score -inf.
template <int NCH, int EPL>
__device__ __forceinline__ void mask_stale_scores(const PairTile<NCH, EPL>& t, int kg,
                                                  float (&s)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = 4 * kg + i < t.lastA ? s[i] : kNegInf;
    s[4 + i] = 4 * kg + i < t.lastB ? s[4 + i] : kNegInf;
  }
}

// Online-softmax update of one N block with the pair's scores s (log2 units, masked ones
// -inf); returns the weights (lifted by kWeightLift) split into the hi / lo P^T operands. The
// exponent of a weight is the difference s - m of two fp32 values, so the weight of a score
// equal to the reference max is exactly 1 (a one-token context returns its value row
// exactly); a fused s * sl2 - m would leave the product's rounding error in that exponent.
template <int KT, int EPL>
__device__ __forceinline__ void softmax_step(WaveState<EPL>& st, const float (&s)[8], uint4& phi,
                                             uint4& plo) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
  mx = row4_max(mx);
  // Lazy rescaling: the reference max moves only when a score exceeds it by more than
  // kRescaleSlack, so weights stay <= 2^kRescaleSlack (times the lift) and the accumulator is
  // rescaled on few steps instead of every step. Any reference value gives the same softmax;
  // the final normalisation divides it out.
  const float mn = fmaxf(st.m_run, mx);
  const bool upd = mn > st.m_run + kRescaleSlack;  // also true while m_run is -inf
  if (__any(upd)) {
    const float m_new = upd ? mn : st.m_run;
    const float alpha = upd ? fast_exp2(st.m_run - (m_new == kNegInf ? 0.f : m_new)) : 1.f;
    st.l_run *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[e] *= alpha;
    st.m_run = m_new;
  }
  const float mu = (st.m_run == kNegInf ? 0.f : st.m_run) - kWeightLift<KT>;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = fast_exp2(s[i] - mu);
  float psum = p[0];  // the same bits as 0 + p[0] (weights are >= 0), one add fewer
#pragma unroll
  for (int i = 1; i < 8; ++i) psum += p[i];
  st.l_run += psum;
  split_weights<KT>(p, phi, plo);
}

// Online softmax and p.V for one loaded pair whose scores s are computed (decode).
template <int KT, int NCH, int EPL>
__device__ __forceinline__ void pair_finish(PairTile<NCH, EPL>& t, WaveState<EPL>& st,
                                            float (&s)[8], int kg) {
  constexpr int BS = 16;
  if (t.lastA < BS || t.lastB < BS) {  // a block holds positions at or past the end
    mask_stale_scores(t, kg, s);
    clear_stale_rows(t, kg);
  }
  uint4 phi, plo;
  softmax_step<KT>(st, s, phi, plo);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const uint4 vt = vt_operand(t, e);
    st.acc[e] = mfma16x16x32<KT>(vt, phi, st.acc[e]);
    st.acc[e] = mfma16x16x32<KT>(vt, plo, st.acc[e]);
  }
}

// q.K, online softmax and p.V for one loaded pair and one 16-row N block (decode).
template <int KT, int NCH, int EPL>
__device__ __forceinline__ void pair_compute(PairTile<NCH, EPL>& t, WaveState<EPL>& st,
                                             const uint4 (&qb)[NCH], float sl2, int kg) {
  float s[8];
  pair_scores<KT>(t, qb, sl2, s);
  pair_finish<KT>(t, st, s, kg);
}

}  // namespace pagedkv
