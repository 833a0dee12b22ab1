// Multi-query causal attention over the paged cache: prefill, chunked prefill and recompute.
//
// Sequence b contributes Q_b query rows, its last Q_b logical positions; query i sits at
// position p = L_b - Q_b + i and attends to positions 0..p through the block table. This is
// the causal attention the Llama engine runs for prefill and recomputation ("vLLM-Style Llama
// Inference Engine with Tensor Parallelism", Features and scope / Implemented; How it works,
// step 4), done over the paged cache as the ragged, padding-free attention over block tables
// that llm-stack's Roadmap plans, with grouped-query heads.
//
// Work decomposition: a workgroup of NW waves takes one KV head g of one sequence and
// NW*NB*R consecutive query tokens; each wave owns NB MFMA N blocks of 16 query rows, each
// block R = 16/G tokens x the G query heads of g. The wave streams the key blocks 0..(its
// last row's position) in pairs, as the decode kernels do (mfma_tiles.h); each loaded pair
// (K tiles and the transposed V operand) serves all NB blocks, with a per-lane causal mask on
// the pairs that reach past the wave's first row. Rows are written normalised.
#include "launch.h"
#include "mfma_tiles.h"

#include <mutex>

namespace pagedkv {

template <int D, int NW, int NB, int MINW, int KT, int OT>
__global__ void __launch_bounds__(NW * 64, MINW)
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
  const int R = 16 / G;  // query tokens per N block
  // Tiles are counted from the end of each sequence and the tile index is the slowest grid
  // dimension, so every sequence's last tile (the one with the most keys under the causal
  // mask) is dispatched first and the light leading tiles fill in behind: a
  // longest-job-first order for the uneven causal work.
  const int unit = blockIdx.x;
  const int bg = unit % (a.batch * Hkv);
  const int tile = unit / (a.batch * Hkv);
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int q0 = a.cu_seqlens_q[b];
  int Q = a.cu_seqlens_q[b + 1] - q0;
  Q = Q < 0 ? 0 : Q;
  const int tok_end = Q - (tile * NW + wave) * NB * R;  // one past this wave's last token
  if (tok_end <= 0) return;                             // no barriers: waves are independent
  const int tok_base = tok_end - NB * R;                // may be negative: rows < 0 are idle
  int L = a.context_lens[b];
  const int Lmax = a.max_blocks * BS;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);

  // Lane row of N block nb: token tok_base + nb*R + n16/G, head n16 % G.
  const int head = n16 % G;
  int tok[NB], row_pos[NB];
  bool row_ok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    tok[nb] = tok_base + nb * R + n16 / G;
    row_ok[nb] = n16 < R * G && tok[nb] >= 0;
    row_pos[nb] = row_ok[nb] ? L - Q + tok[nb] : -1;  // < 0: no key (only when Q > L)
  }
  const int first_tok = tok_base > 0 ? tok_base : 0;
  const int p_min = L - Q + first_tok;
  const int p_max = L - Q + tok_end - 1;
  const int tok1 = p_max + 1 > 0 ? p_max + 1 : 0;  // keys 0 .. tok1-1 can matter to this wave
  const int blk1 = (tok1 + BS - 1) / BS;

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
          pair_compute_nb<KT>(t[u], st, qb, sl2, kg, row_pos, key0, key0 + 2 * BS - 1 > p_min);
        }
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l_run = st[nb].l_run;
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    if (row_ok[nb]) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      const size_t o = ((size_t)(q0 + tok[nb]) * Hq + (size_t)g * G + head) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          store_out4<OT>(a.out, o + EPL * (4 * kg + i) + e, st[nb].acc[e][i] * inv,
                         st[nb].acc[e + 1][i] * inv, st[nb].acc[e + 2][i] * inv,
                         st[nb].acc[e + 3][i] * inv);
    }
  }
}

bool supported_prefill(int head_dim, int group, int block_size) {
  return block_size == 16 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

int prefill_tokens_per_group(int group, int nb) { return kWavesPerGroup * nb * (16 / group); }

// Register use (and so occupancy) is taken from the bf16 -> fp32 instance of each (D, NB);
// the other formats differ only in conversions and the output store.
template <int D, int NB>
static const void* prefill_kernel_ptr() {
  return reinterpret_cast<const void*>(
      &prefill_mfma_kernel<D, kWavesPerGroup, NB, NB == 1 ? 2 : 1, kDtBf16, kDtF32>);
}

// Workgroups of the (D, NB) variant one CU holds at once, asked of the runtime once per
// device (it follows from the variant's register count).
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

// N blocks of 16 query rows per wave (1, 2 or 4). A larger NB reuses every loaded key/value
// pair for more rows but holds more registers, so fewer workgroups fit on a CU, and it cuts
// the query rows into fewer workgroups. The launch takes the largest NB whose workgroups
// (counted from the total query rows, a lower bound for ragged batches) still fill the
// resident slots at least twice, so the longest-first order can balance them. NB stops at 2
// for head_dim 64: there NB = 4 drops the variant from two waves per SIMD to one, which
// measured slower than the extra reuse gains; at head_dim 128 NB = 2 and 4 both hold one wave
// per SIMD. A build may pin NB with PAGEDKV_PREFILL_NB.
int prefill_rows_per_wave(int64_t num_tokens, int num_kv_heads, int head_dim, int group,
                          int cus) {
#ifdef PAGEDKV_PREFILL_NB
  (void)num_tokens; (void)num_kv_heads; (void)head_dim; (void)group; (void)cus;
  return PAGEDKV_PREFILL_NB;
#else
  const int max_index = head_dim >= 128 ? 2 : 1;
  for (int i = max_index; i > 0; --i) {
    const int nb = 1 << i;
    const int64_t per_group = prefill_tokens_per_group(group, nb);
    const int64_t units = (int64_t)num_kv_heads * ((num_tokens + per_group - 1) / per_group);
    const int64_t slots = (int64_t)cus * prefill_groups_per_cu(head_dim, i);
    if (units >= 2 * slots) return nb;
  }
  return 1;
#endif
}

template <int D, int KT, int OT>
static hipError_t launch_prefill_d(const PrefillArgs& a, unsigned grid, hipStream_t stream) {
  constexpr int NW = kWavesPerGroup;
  switch (a.nb) {
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 1, 2, KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 2, 1, KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<D, NW, 4, 1, KT, OT>), dim3(grid), dim3(NW * 64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)((long long)a.batch * a.num_kv_heads * a.ntiles);
  return with_formats(a.kv_dtype, a.out_dtype, [&](auto kt, auto ot) {
    constexpr int KT = decltype(kt)::value, OT = decltype(ot)::value;
    if (a.head_dim == 128) return launch_prefill_d<128, KT, OT>(a, units, stream);
    if (a.head_dim == 64) return launch_prefill_d<64, KT, OT>(a, units, stream);
    return hipErrorInvalidValue;
  });
}

}  // namespace pagedkv
