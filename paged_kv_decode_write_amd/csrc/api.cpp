// C-ABI host layer of libpagedkv: argument validation, status codes, the partition plan and
// kernel dispatch. Declarations and the contract of every entry point: include/paged_kv.h.
#include "paged_kv.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "launch.h"

using namespace pagedkv;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PAGEDKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Compute-unit count of the current device, queried once per device. PAGEDKV_CU_COUNT (a
// positive integer) replaces the query, so the host-side planning can be exercised without a
// device.
int cu_count(int* out) {
  if (const char* env = std::getenv("PAGEDKV_CU_COUNT")) {
    const long n = std::strtol(env, nullptr, 10);
    if (n > 0 && n < (1L << 20)) {
      *out = (int)n;
      return PAGEDKV_OK;
    }
  }
  static std::mutex mu;
  static int counts[256] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 256) return fail(PAGEDKV_ERR_HIP, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (counts[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    counts[dev] = n > 0 ? n : 1;
  }
  *out = counts[dev];
  return PAGEDKV_OK;
}

// Smallest partition the automatic choice makes, in tokens. Partitions shorter than this
// spend more on the per-partition set-up and merge than they gain in parallelism.
constexpr int64_t kMinAutoPartition = 256;
// Work the automatic choice aims for, per compute unit: workgroups of the kernels that split
// a partition over a workgroup's waves; waves of the kernel with one wave per KV head (two
// per SIMD, one full residency round). With few (sequence, KV head) units, i.e. few long
// contexts, that kernel aims for one wave per SIMD instead: fewer, longer partitions, which
// measured faster there (less per-wave start-up, a smaller merge).
constexpr int64_t kTargetGroupsPerCU = 4;
constexpr int64_t kTargetHeadWavesPerCU = 8;
constexpr int64_t kTargetHeadWavesPerCUFewUnits = 4;
// Contexts longer than this many tokens use the one-wave-per-KV-head kernel by default;
// shorter ones spread each partition over a workgroup's waves for lower latency.
constexpr int64_t kHeadWaveMinContext = 1024;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

struct Plan {
  int32_t nparts;
  int32_t part_tokens;
};

// Partition plan. max_len = MB * block_size bounds every context length; the plan never
// reads context_lens (that would need a device-to-host copy and a sync).
// `granule`: automatic partitions are rounded up to a multiple of this many tokens (the
// tokens one workgroup step covers: waves x blocks per wave step x block_size).
int make_plan(int32_t batch, int32_t num_kv_heads, int32_t max_blocks, int32_t block_size,
              int32_t partition_tokens, int cus, int kernel, int granule, Plan* plan) {
  const int64_t max_len = (int64_t)max_blocks * block_size;
  if (partition_tokens < -1) return fail(PAGEDKV_ERR_SHAPE, "partition_tokens must be >= -1");
  int64_t n = 1, P = 0;
  if (partition_tokens == -1 || max_len == 0) {
    n = 1;
  } else if (partition_tokens > 0) {
    if (partition_tokens % block_size)
      return fail(PAGEDKV_ERR_SHAPE, "partition_tokens %d is not a multiple of block_size %d",
                  partition_tokens, block_size);
    P = partition_tokens;
    n = ceil_div(max_len, P);
  } else {
    const int64_t units = (int64_t)batch * num_kv_heads;
    int64_t target = kTargetGroupsPerCU * cus;
    if (kernel == PAGEDKV_KERNEL_MFMA_HEADWAVE)
      target = (units * 4 <= cus ? kTargetHeadWavesPerCUFewUnits : kTargetHeadWavesPerCU) * cus;
    const int64_t nmax = ceil_div(max_len, kMinAutoPartition);
    n = units > 0 ? ceil_div(target, units) : 1;
    if (n > nmax) n = nmax;
    if (n < 1) n = 1;
    P = round_up(ceil_div(max_len, n), (int64_t)granule);
    n = ceil_div(max_len, P);
  }
  if (n <= 1) {
    n = 1;
    P = max_len > 0 ? round_up(max_len, block_size) : block_size;
  }
  if (P > INT32_MAX || n > INT32_MAX) return fail(PAGEDKV_ERR_SHAPE, "partition plan overflows");
  if ((int64_t)batch * num_kv_heads * n > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE, "too many workgroups (batch * kv heads * partitions)");
  plan->nparts = (int32_t)n;
  plan->part_tokens = (int32_t)P;
  return PAGEDKV_OK;
}

// Evenly divided (stream-K) decode. A workgroup takes at least `min_pairs` 32-token pairs of
// the batch's work, so a (sequence, KV head) whose pairs_max pairs at most fall to workgroups
// in slices of q >= min_pairs items touches at most (pairs_max - 1) / min_pairs + 2 of them:
// that many partial slots. Automatically the slots are at most kStreamSlots (min_pairs from the
// table width alone, so the workspace bound needs no device; and never below 256 tokens, below
// which a slice costs more in start-up than it gains in balance); partition_tokens > 0 sets
// min_pairs to that many tokens instead. The grid is one workgroup (four waves, one per SIMD)
// per compute unit: with two resident per CU (the registers allow two), the second one's
// loads were served only after most of the first one's, so on a ragged batch the second
// finished a quarter of the dispatch later, and the whole kernel ran 5-6% slower.
constexpr int64_t kStreamSlots = 16;
constexpr int64_t kStreamPairTokens = 32;
constexpr int kStreamGroupsPerCU = 1;
// Compute units of a whole MI355X / MI350X (8 XCDs of 32), where the stream kernel weights its
// slices by XCD (see decode_sk.hip).
constexpr int kXcdWeightedCUs = 256;

struct StreamPlan {
  int32_t min_pairs;
  int32_t slots;
};

StreamPlan stream_plan(int64_t max_len, int32_t partition_tokens) {
  const int64_t pairs_max = ceil_div(max_len, kStreamPairTokens);
  int64_t q = 1;
  if (partition_tokens > 0) {
    q = ceil_div(partition_tokens, kStreamPairTokens);
  } else {
    q = kMinAutoPartition / kStreamPairTokens;  // automatic slices stay >= 256 tokens
    if (pairs_max > 1 && ceil_div(pairs_max - 1, kStreamSlots - 2) > q)
      q = ceil_div(pairs_max - 1, kStreamSlots - 2);
  }
  if (q < 1) q = 1;
  const int64_t slots = pairs_max > 0 ? (pairs_max - 1) / q + 2 : 2;
  return StreamPlan{(int32_t)q, (int32_t)slots};
}

// Upper bound of the partition count for a partition_tokens setting, device-independent.
// (The stream family serves contexts over kHeadWaveMinContext tokens only, so its slots count
// only there.)
int64_t nparts_bound(int64_t max_len, int32_t block_size, int32_t partition_tokens) {
  if (max_len <= 0 || partition_tokens == -1) return 1;
  if (partition_tokens > 0 && partition_tokens % block_size) return 1;
  const int64_t n = ceil_div(max_len, partition_tokens > 0 ? partition_tokens : kMinAutoPartition);
  if (max_len <= kHeadWaveMinContext) return n;
  const int64_t s = stream_plan(max_len, partition_tokens).slots;
  return n > s ? n : s;
}

// Workspace layout of a split call: [partial outputs | partial (max, sum)].
size_t acc_bytes(int64_t B, int64_t Hq, int64_t D, int64_t n) {
  return (size_t)round_up(B * Hq * n * D * 4, 256);
}

size_t split_workspace_bytes(int64_t B, int64_t Hq, int64_t D, int64_t n) {
  if (n <= 1) return 0;
  return acc_bytes(B, Hq, D, n) + (size_t)round_up(B * Hq * n * 2 * 4, 256);
}

// Blocks larger than 16 tokens. The decode kernels are built for 16-token blocks; a pool of
// blocks of 16 * sub tokens is the same memory as a pool of 16-token blocks (block p is
// 16-token blocks sub * p .. sub * p + sub - 1, and slot numbers name the same rows), so a
// call with larger blocks attends over that view, through a table of 16-token block ids that
// one small launch writes into the workspace, after the split region.
constexpr int32_t kKernelBlock = 16;
constexpr int32_t kMaxDecodeBlock = 1024;

int decode_block_view(int32_t block_size, int32_t* sub) {
  if (block_size % kKernelBlock || block_size > kMaxDecodeBlock)
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "block_size %d: decode attention takes a multiple of 16 up to %d", block_size,
                (int)kMaxDecodeBlock);
  *sub = block_size / kKernelBlock;
  return PAGEDKV_OK;
}

size_t view_table_bytes(int64_t batch, int64_t max_blocks, int32_t sub) {
  return sub > 1 ? (size_t)round_up(batch * max_blocks * sub * 4, 256) : 0;
}

// Key split of the multi-query kernel. It pays when the batch's query tiles are too few to
// fill the device and contexts are long: one tile's keys are then a long serial chain that a
// few workgroups walk while the rest of the device idles. The automatic choice splits when the
// workgroups that have rows to compute (counted from num_tokens, a lower bound for ragged
// batches) fill fewer than two residency rounds and the contexts may exceed
// kPrefillSplitMinKeys; it cuts them into at most kPrefillMaxAutoParts partitions of at least
// kPrefillMinPartKeys keys. Partitions are multiples of the 32 keys one staged pair holds.
// Three partitions measured best on the ragged mix of short chunks and full prefills up to
// 4000 keys (75 us per call, against 87 with four partitions of 1024 keys and 93 with two of
// 2048): each split workgroup pays its start (block ids, the first staged pair) once, and a
// fourth partition adds more workgroups and merge input than it removes from the longest
// chain.
constexpr int64_t kPrefillSplitMinKeys = 2048;
constexpr int64_t kPrefillMaxAutoParts = 3;
constexpr int64_t kPrefillMinPartKeys = 512;
constexpr int64_t kPrefillPairKeys = 32;
// Workgroups of the one- and two-block kernels one CU holds (their registers allow two); a
// constant so that the split does not depend on an occupancy query.
constexpr int64_t kPrefillGroupsPerCU = 2;

struct PrefillPlan {
  int32_t nb;         // 16-row blocks per wave
  int32_t nparts;     // key partitions per query tile
  int32_t part_keys;  // keys per partition
  int64_t ntiles;     // query tiles per sequence
};

int64_t prefill_auto_part_keys(int64_t max_len) {
  const int64_t P = round_up(ceil_div(max_len, kPrefillMaxAutoParts), kPrefillPairKeys);
  return P > kPrefillMinPartKeys ? P : kPrefillMinPartKeys;
}

// Upper bound of the partition count, device-independent (sizes the workspace).
int64_t prefill_nparts_bound(int64_t max_len, int32_t partition_tokens) {
  if (max_len <= 0 || partition_tokens == -1) return 1;
  if (partition_tokens > 0)
    return partition_tokens % kPrefillPairKeys ? 1 : ceil_div(max_len, partition_tokens);
  if (max_len <= kPrefillSplitMinKeys) return 1;
  return ceil_div(max_len, prefill_auto_part_keys(max_len));
}

int check_prefill_knobs(int32_t row_blocks, int32_t partition_tokens) {
  if (row_blocks != 0 && row_blocks != 1 && row_blocks != 2 && row_blocks != 4)
    return fail(PAGEDKV_ERR_SHAPE, "row_blocks must be 0 (auto), 1, 2 or 4, got %d", row_blocks);
  if (partition_tokens < -1)
    return fail(PAGEDKV_ERR_SHAPE, "partition_tokens must be >= -1");
  if (partition_tokens > 0 && partition_tokens % kPrefillPairKeys)
    return fail(PAGEDKV_ERR_SHAPE, "partition_tokens %d is not a multiple of %d",
                partition_tokens, (int)kPrefillPairKeys);
  return PAGEDKV_OK;
}

int make_prefill_plan(int64_t num_tokens, int32_t max_q_len, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int G,
                      int32_t max_blocks, int32_t block_size, int32_t row_blocks,
                      int32_t partition_tokens, int cus, PrefillPlan* plan) {
  const int st = check_prefill_knobs(row_blocks, partition_tokens);
  if (st) return st;
  const int nb = row_blocks > 0 ? row_blocks
                                : prefill_rows_per_wave(num_tokens, num_kv_heads, head_dim, G, cus);
  const int64_t per_group = prefill_tokens_per_group(G, nb);
  const int64_t ntiles = ceil_div(max_q_len, per_group);
  const int64_t max_len = (int64_t)max_blocks * block_size;
  const bool rows_fit = num_tokens * num_q_heads <= INT32_MAX;  // the merge's row count
  int64_t n = 1, P = 0;
  if (partition_tokens > 0 && max_len > 0) {
    P = partition_tokens;
    n = ceil_div(max_len, P);
    if (n > 1 && !rows_fit)
      return fail(PAGEDKV_ERR_SHAPE, "num_tokens * num_q_heads exceeds int32 for a key split");
  } else if (partition_tokens == 0 && max_len > kPrefillSplitMinKeys && rows_fit) {
    const int64_t groups = (int64_t)num_kv_heads * ceil_div(num_tokens, per_group);
    if (groups < 2 * kPrefillGroupsPerCU * cus) {
      P = prefill_auto_part_keys(max_len);
      n = ceil_div(max_len, P);
    }
  }
  if (n <= 1) {
    n = 1;
    P = round_up(max_len > 0 ? max_len : 1, kPrefillPairKeys);
  }
  if (P > INT32_MAX) return fail(PAGEDKV_ERR_SHAPE, "partition plan overflows");
  if ((int64_t)batch * num_kv_heads * ntiles * n > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE,
                "too many workgroups (batch * kv heads * query tiles * key partitions)");
  plan->nb = nb;
  plan->nparts = (int32_t)n;
  plan->part_keys = (int32_t)P;
  plan->ntiles = ntiles;
  return PAGEDKV_OK;
}

int select_kernel(int32_t kernel, int D, int G, int bs, int64_t max_len, int* chosen) {
  switch (kernel) {
    case PAGEDKV_KERNEL_AUTO:
      if (supported_mfma(D, G, bs)) {
        *chosen = max_len > kHeadWaveMinContext ? PAGEDKV_KERNEL_MFMA_HEADWAVE : PAGEDKV_KERNEL_MFMA;
        return PAGEDKV_OK;
      }
      if (supported_valu(D, G, bs)) { *chosen = PAGEDKV_KERNEL_VALU; return PAGEDKV_OK; }
      break;
    case PAGEDKV_KERNEL_VALU:
      if (supported_valu(D, G, bs)) { *chosen = kernel; return PAGEDKV_OK; }
      break;
    case PAGEDKV_KERNEL_MFMA:
    case PAGEDKV_KERNEL_MFMA_HEADWAVE:
    case PAGEDKV_KERNEL_MFMA_STREAM:
      if (supported_mfma(D, G, bs)) { *chosen = kernel; return PAGEDKV_OK; }
      break;
    default:
      return fail(PAGEDKV_ERR_UNSUPPORTED, "unknown kernel family %d", kernel);
  }
  return fail(PAGEDKV_ERR_UNSUPPORTED,
              "no %s kernel for head_dim %d, block_size %d, group size %d",
              kernel == PAGEDKV_KERNEL_MFMA ? "MFMA" : kernel == PAGEDKV_KERNEL_VALU ? "VALU" : "",
              D, bs, G);
}

// The launch of a decode call: the kernel family, its partitions (for the stream family:
// partial slots and minimum tokens per workgroup) and, for the stream family, the grid.
// An automatic choice of the head-per-wave kernel becomes the stream family when the caller
// left the split to the library, the (sequence, KV head) units exceed a quarter of the compute
// units, and the head-per-wave plan has more workgroups than compute units. The head-per-wave
// plan then keeps two workgroups on a compute unit, and the second one's loads are served
// mostly after the first one's: it finishes a quarter of the dispatch later, with its compute
// unit half idle meanwhile; on a ragged batch the plan also leaves partitions empty or short.
// The stream family runs one workgroup per compute unit on equal slices and measured faster
// on ragged batches (13%) and on uniform long ones (1.5%). With fewer workgroups than compute
// units (few, short contexts) the head-per-wave kernel stays: the stream family's extra
// memory round trip (it reads the lengths before it can read the block ids) costs more there
// than the balance gains (10% on 16 x 2048 tokens of head_dim 64). The host cannot see the
// lengths without reading context_lens, which would need a synchronisation.
struct DecodePlan {
  int kernel;
  Plan plan;
  int32_t min_pairs;  // stream family only
  int32_t grid;       // stream family only
};

int plan_granule(int kernel, int32_t block_size);

int plan_decode(int32_t requested, int chosen, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t mb16, int32_t partition_tokens, int cus,
                DecodePlan* out) {
  const int64_t units = (int64_t)batch * num_kv_heads;
  if (requested == PAGEDKV_KERNEL_AUTO && chosen == PAGEDKV_KERNEL_MFMA_HEADWAVE &&
      partition_tokens == 0 && units * 4 > cus) {
    Plan hw{};
    const int st = make_plan(batch, num_kv_heads, mb16, kKernelBlock, 0, cus, chosen,
                             plan_granule(chosen, kKernelBlock), &hw);
    if (st) return st;
    const int64_t groups = (int64_t)batch * ceil_div(num_kv_heads, kHeadsPerGroup) * hw.nparts;
    if (groups > cus) chosen = PAGEDKV_KERNEL_MFMA_STREAM;
  }
  out->kernel = chosen;
  out->min_pairs = 0;
  out->grid = 0;
  if (chosen != PAGEDKV_KERNEL_MFMA_STREAM)
    return make_plan(batch, num_kv_heads, mb16, kKernelBlock, partition_tokens, cus, chosen,
                     plan_granule(chosen, kKernelBlock), &out->plan);
  if ((int64_t)mb16 * kKernelBlock <= kHeadWaveMinContext)
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "the stream kernel family takes contexts over %d tokens (max_blocks_per_seq * "
                "block_size)", (int)kHeadWaveMinContext);
  if (partition_tokens == -1)
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "the stream kernel family always leaves partials (partition_tokens -1)");
  if (partition_tokens < -1) return fail(PAGEDKV_ERR_SHAPE, "partition_tokens must be >= -1");
  if (partition_tokens > 0 && partition_tokens % kKernelBlock)
    return fail(PAGEDKV_ERR_SHAPE, "partition_tokens %d is not a multiple of 16",
                partition_tokens);
  const int64_t max_len = (int64_t)mb16 * kKernelBlock;
  const StreamPlan sp = stream_plan(max_len, partition_tokens);
  const int64_t ngrp = ceil_div(num_kv_heads, kHeadsPerGroup);
  const int64_t work = (int64_t)batch * ngrp * ceil_div(max_len, kStreamPairTokens);
  const int64_t grid = (int64_t)kStreamGroupsPerCU * cus;
  if (work + grid > INT32_MAX / 2 || grid > INT32_MAX / 2 ||
      (int64_t)batch * num_q_heads * sp.slots > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE, "stream plan overflows (batch * heads * context too large)");
  out->plan.nparts = sp.slots;
  out->plan.part_tokens = (int32_t)(sp.min_pairs * kStreamPairTokens);
  out->min_pairs = sp.min_pairs;
  out->grid = (int32_t)grid;
  return PAGEDKV_OK;
}

int plan_granule(int kernel, int32_t block_size) {
  switch (kernel) {
    case PAGEDKV_KERNEL_MFMA: return kWavesPerGroup * block_size * 2;
    case PAGEDKV_KERNEL_MFMA_HEADWAVE: return block_size * 2;
    default: return kWavesPerGroup * block_size;
  }
}

int check_formats(int32_t kv_dtype, int32_t out_dtype) {
  if (kv_dtype != PAGEDKV_DTYPE_BF16 && kv_dtype != PAGEDKV_DTYPE_F16)
    return fail(PAGEDKV_ERR_UNSUPPORTED, "q and cache format %d is not bf16 or fp16", kv_dtype);
  if (out_dtype != PAGEDKV_DTYPE_F32 && out_dtype != kv_dtype)
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "output format %d: fp32 or the input format (%d) are supported", out_dtype,
                kv_dtype);
  return PAGEDKV_OK;
}

int check_decode_sizes(int32_t max_blocks, int32_t batch, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks) {
  if (batch < 0 || max_blocks < 0)
    return fail(PAGEDKV_ERR_SHAPE, "batch and max_blocks_per_seq must be >= 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PAGEDKV_ERR_SHAPE, "head counts, head_dim, block_size, num_blocks must be > 0");
  if (num_q_heads % num_kv_heads)
    return fail(PAGEDKV_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if ((int64_t)max_blocks * block_size > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE, "max_blocks_per_seq * block_size exceeds int32");
  return PAGEDKV_OK;
}

// The KV write of a fused decode step: token b's rows go to slot_mapping[b] of the pools;
// with positions non-null, q and k_new are first rotated at positions[b] (rotated q to q_out).
struct StepWrite {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* slot_mapping;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* positions;
  const float* inv_freq;
  int32_t interleaved;
  uint16_t* q_out;
};

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Scratch of paged_decode_step_noalloc: the split partials and the block-table view of a decode
// call, in a file-scope device array instead of a caller's workspace. Each device holds its own
// copy for the life of the process; calls on one device share it (see the header).
static __device__ __align__(256) unsigned char scratch[PAGEDKV_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device with that device
// current and kept; host code uses this address, never the array's name (which in host code
// is a stand-in, not a device address).
int scratch_address(void** out) {
  static std::mutex mu;
  static void* ptrs[256] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 256) return fail(PAGEDKV_ERR_HIP, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PAGEDKV_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return PAGEDKV_OK;
}

// Decode attention, optionally fused with the step's KV write (sw non-null).
// The checked build (PAGEDKV_CHECKED) validates a call's data on the device before its
// kernels, on the same stream; the unchecked build launches nothing here.
#ifdef PAGEDKV_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

int check_slots(const int64_t* slots, int64_t n, int64_t num_slots, hipStream_t stream) {
  if (!kChecked) return PAGEDKV_OK;
  const hipError_t e = launch_check_slots(slots, n, num_slots, stream);
  return e == hipSuccess ? PAGEDKV_OK : hip_fail(e, "slot check launch");
}

int check_tables(const int32_t* tables, const int32_t* lens, int32_t batch, int32_t max_blocks,
                 int32_t block_size, int64_t num_blocks, hipStream_t stream) {
  if (!kChecked) return PAGEDKV_OK;
  const hipError_t e =
      launch_check_tables(tables, lens, batch, max_blocks, block_size, num_blocks, stream);
  return e == hipSuccess ? PAGEDKV_OK : hip_fail(e, "block table check launch");
}

int check_queries(const int32_t* cu, const int32_t* lens, int32_t batch, int32_t max_blocks,
                  int32_t block_size, int64_t num_tokens, int32_t max_q_len,
                  hipStream_t stream) {
  if (!kChecked) return PAGEDKV_OK;
  const hipError_t e = launch_check_queries(cu, lens, batch, max_blocks, block_size, num_tokens,
                                            max_q_len, stream);
  return e == hipSuccess ? PAGEDKV_OK : hip_fail(e, "query span check launch");
}

int decode_impl(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                float scale, int32_t kv_dtype, void* out, int32_t out_dtype, void* workspace,
                size_t workspace_bytes, int32_t partition_tokens, int32_t kernel,
                hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream,
                const StepWrite* sw, bool static_scratch = false) {
  g_last_error.clear();
  int st = check_formats(kv_dtype, out_dtype);
  if (st) return st;
  st = check_decode_sizes(max_blocks_per_seq, batch, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks);
  if (st) return st;
  int32_t sub = 1;
  st = decode_block_view(block_size, &sub);
  if (st) return st;
  if (sub > 1 && partition_tokens > 0 && partition_tokens % block_size)
    return fail(PAGEDKV_ERR_SHAPE, "partition_tokens %d is not a multiple of block_size %d",
                partition_tokens, block_size);
  if (num_blocks > (int64_t)INT32_MAX / sub)
    return fail(PAGEDKV_ERR_SHAPE, "num_blocks * block_size / 16 exceeds int32");
  // From here on, sizes are those of the 16-token view.
  const int32_t mb16 = max_blocks_per_seq * sub;
  const int64_t nb16 = num_blocks * sub;
  const int G = num_q_heads / num_kv_heads;
  int chosen = 0;
  st = select_kernel(kernel, head_dim, G, kKernelBlock, (int64_t)mb16 * kKernelBlock, &chosen);
  if (st) return st;
  if (batch == 0) return PAGEDKV_OK;
  if (!q || !k_cache || !v_cache || !context_lens || !out ||
      (max_blocks_per_seq > 0 && !block_tables))
    return fail(PAGEDKV_ERR_NULL,
                "q, k_cache, v_cache, block_tables, context_lens and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PAGEDKV_ERR_ALIGN, "q, k_cache, v_cache and out need 16-byte alignment");
  if (sw) {
    if (!sw->k_new || !sw->v_new || !sw->slot_mapping)
      return fail(PAGEDKV_ERR_NULL, "k_new, v_new and slot_mapping must be non-NULL");
    if (!aligned(sw->k_new, 16) || !aligned(sw->v_new, 16) || !aligned(sw->slot_mapping, 8))
      return fail(PAGEDKV_ERR_ALIGN, "k_new and v_new need 16-byte alignment");
    if (sw->positions) {
      if (kv_dtype != PAGEDKV_DTYPE_BF16)
        return fail(PAGEDKV_ERR_UNSUPPORTED, "the rotary decode step takes bf16 inputs only");
      if (sw->interleaved != 0 && sw->interleaved != 1)
        return fail(PAGEDKV_ERR_SHAPE, "interleaved must be 0 or 1");
      if (!sw->inv_freq || !sw->q_out)
        return fail(PAGEDKV_ERR_NULL, "positions, inv_freq and q_out must be non-NULL");
      if (!aligned(sw->inv_freq, 16) || !aligned(sw->q_out, 16) || !aligned(sw->positions, 4))
        return fail(PAGEDKV_ERR_ALIGN, "inv_freq and q_out need 16-byte alignment");
      const size_t qbytes = (size_t)batch * num_q_heads * head_dim * 2;
      if (ranges_overlap(q, qbytes, sw->q_out, qbytes))
        return fail(PAGEDKV_ERR_SHAPE, "q_out must not overlap q");
    }
  }
  int cus = 0;
  st = cu_count(&cus);
  if (st) return st;
  DecodePlan dp{};
  st = plan_decode(kernel, chosen, batch, num_q_heads, num_kv_heads, mb16, partition_tokens, cus,
                   &dp);
  if (st) return st;
  chosen = dp.kernel;
  const Plan plan = dp.plan;

  DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.max_blocks = mb16;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = kKernelBlock;
  a.num_blocks = nb16;
  a.scale_log2 = scale * kLog2eHost;
  a.nparts = plan.nparts;
  a.part_tokens = plan.part_tokens;
  a.kv_dtype = kv_dtype;
  a.out_dtype = out_dtype;
  a.sk_min_pairs = dp.min_pairs;
  // The stream family's XCD-weighted slices assume the whole device: 8 XCDs of 32 CUs, to
  // which the dispatcher deals workgroups in turn.
  a.sk_xcd_weights = chosen == PAGEDKV_KERNEL_MFMA_STREAM && cus == kXcdWeightedCUs;
  const size_t split_need = split_workspace_bytes(batch, num_q_heads, head_dim, plan.nparts);
  const size_t table_need = view_table_bytes(batch, max_blocks_per_seq, sub);
  if (static_scratch) {
    const size_t need = split_need + table_need;
    if (need > PAGEDKV_STATIC_SCRATCH_BYTES)
      return fail(PAGEDKV_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch (%d partitions of %d tokens); the "
                  "static scratch holds %zu (PAGEDKV_STATIC_SCRATCH_BYTES)",
                  need, plan.nparts, plan.part_tokens, (size_t)PAGEDKV_STATIC_SCRATCH_BYTES);
    st = scratch_address(&workspace);
    if (st) return st;
    workspace_bytes = PAGEDKV_STATIC_SCRATCH_BYTES;
  }
  if (split_need + table_need > 0) {
    const size_t need = split_need + table_need;
    if (!workspace || workspace_bytes < need)
      return fail(PAGEDKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(PAGEDKV_ERR_ALIGN, "workspace needs 16-byte alignment");
  }
  char* base = static_cast<char*>(workspace);
  if (plan.nparts > 1) {
    a.ws_acc = reinterpret_cast<float*>(base);
    a.ws_ml = reinterpret_cast<float*>(base + acc_bytes(batch, num_q_heads, head_dim, plan.nparts));
  }

  st = check_tables(block_tables, context_lens, batch, max_blocks_per_seq, block_size,
                    num_blocks, stream);
  if (st) return st;
  if (sw) {
    st = check_slots(sw->slot_mapping, batch, num_blocks * block_size, stream);
    if (st) return st;
  }
  hipError_t e;
  if (sw && chosen == PAGEDKV_KERNEL_VALU && sw->positions) {
    // The vector-ALU kernel has no fused write: rotate and store first, then attend over the
    // pools with the rotated q.
    RopeArgs r{};
    r.q = q;
    r.k = sw->k_new;
    r.v = sw->v_new;
    r.positions = sw->positions;
    r.inv_freq = sw->inv_freq;
    r.slot_mapping = sw->slot_mapping;
    r.q_out = sw->q_out;
    r.k_cache = sw->k_cache;
    r.v_cache = sw->v_cache;
    r.num_tokens = batch;
    r.num_slots = num_blocks * block_size;
    r.num_q_heads = num_q_heads;
    r.num_kv_heads = num_kv_heads;
    r.head_dim = head_dim;
    r.interleaved = sw->interleaved;
    e = launch_kv_write_rope(r, stream);
    if (e != hipSuccess) return hip_fail(e, "rope + kv_write launch");
    a.q = sw->q_out;
  } else if (sw && chosen == PAGEDKV_KERNEL_VALU) {
    // The vector-ALU kernel has no fused write: store first, then attend over the pools.
    e = launch_kv_write(sw->k_new, sw->v_new, sw->slot_mapping, batch, sw->k_cache,
                        sw->v_cache, num_blocks * block_size, num_kv_heads * head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "kv_write launch");
  } else if (sw) {
    a.k_new = sw->k_new;
    a.v_new = sw->v_new;
    a.slot_mapping = sw->slot_mapping;
    a.k_cache_w = sw->k_cache;
    a.v_cache_w = sw->v_cache;
    a.positions = sw->positions;
    a.inv_freq = sw->inv_freq;
    a.interleaved = sw->interleaved;
    a.q_out = sw->q_out;
  }
  if (sub > 1) {
    int32_t* view = reinterpret_cast<int32_t*>(base + split_need);
    e = launch_expand_table(block_tables, batch, max_blocks_per_seq, sub, num_blocks, view,
                            stream);
    if (e != hipSuccess) return hip_fail(e, "block table view launch");
    a.block_tables = view;
  }
  if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess)
    return hip_fail(e, "hipEventRecord(begin)");
  switch (chosen) {
    case PAGEDKV_KERNEL_MFMA: e = launch_decode_mfma(a, stream); break;
    case PAGEDKV_KERNEL_MFMA_HEADWAVE: e = launch_decode_mfma_hw(a, stream); break;
    case PAGEDKV_KERNEL_MFMA_STREAM: e = launch_decode_mfma_sk(a, dp.grid, stream); break;
    default: e = launch_decode_valu(a, stream); break;
  }
  if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  if (ev_end && (e = hipEventRecord(ev_end, stream)) != hipSuccess)
    return hip_fail(e, "hipEventRecord(end)");
  if (plan.nparts > 1) {
    e = launch_decode_reduce(a, stream);
    if (e != hipSuccess) return hip_fail(e, "partition merge launch");
  }
  return PAGEDKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_abi_version(void) { return PAGED_KV_ABI_VERSION; }

const char* paged_kv_status_string(int status) {
  switch (status) {
    case PAGEDKV_OK: return "PAGEDKV_OK";
    case PAGEDKV_ERR_NULL: return "PAGEDKV_ERR_NULL";
    case PAGEDKV_ERR_SHAPE: return "PAGEDKV_ERR_SHAPE";
    case PAGEDKV_ERR_UNSUPPORTED: return "PAGEDKV_ERR_UNSUPPORTED";
    case PAGEDKV_ERR_WORKSPACE: return "PAGEDKV_ERR_WORKSPACE";
    case PAGEDKV_ERR_HIP: return "PAGEDKV_ERR_HIP";
    case PAGEDKV_ERR_ALIGN: return "PAGEDKV_ERR_ALIGN";
    default: return "PAGEDKV_UNKNOWN_STATUS";
  }
}

const char* paged_kv_last_error(void) { return g_last_error.c_str(); }

int paged_kv_checked_build(void) { return kChecked ? 1 : 0; }

int paged_kv_check_status(int32_t* code, int64_t* index, int64_t* value, int32_t clear) {
  g_last_error.clear();
  if (!kChecked)
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "this library does not validate data on the device (build with PAGEDKV_CHECKED)");
  if (!code) return fail(PAGEDKV_ERR_NULL, "code must be non-NULL");
  long long rec[3] = {0, 0, 0};
  const hipError_t e = read_check_record(rec, clear != 0);
  if (e != hipSuccess) return hip_fail(e, "reading the check record");
  *code = (int32_t)rec[0];
  if (index) *index = rec[1];
  if (value) *value = rec[2];
  return PAGEDKV_OK;
}

int paged_kv_write(const uint16_t* k, const uint16_t* v, const int64_t* slot_mapping,
                   int64_t num_tokens, uint16_t* k_cache, uint16_t* v_cache,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0) return fail(PAGEDKV_ERR_SHAPE, "num_tokens must be >= 0");
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PAGEDKV_ERR_SHAPE, "num_blocks, block_size, num_kv_heads, head_dim must be > 0");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row % 8)
    return fail(PAGEDKV_ERR_UNSUPPORTED, "num_kv_heads*head_dim (%lld) must be a multiple of 8",
                (long long)row);
  if (row > INT32_MAX) return fail(PAGEDKV_ERR_SHAPE, "row too long");
  if (num_blocks > INT64_MAX / block_size / row)
    return fail(PAGEDKV_ERR_SHAPE, "pool size overflows");
  if (num_tokens == 0) return PAGEDKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PAGEDKV_ERR_NULL, "k, v, slot_mapping, k_cache and v_cache must be non-NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return fail(PAGEDKV_ERR_ALIGN, "k, v, k_cache, v_cache need 16-byte alignment");
  const int st = check_slots(slot_mapping, num_tokens, num_blocks * block_size, stream);
  if (st) return st;
  hipError_t e = launch_kv_write(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                 num_blocks * block_size, (int32_t)row, stream);
  if (e != hipSuccess) return hip_fail(e, "kv_write launch");
  return PAGEDKV_OK;
}

int paged_kv_write_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* positions, const float* inv_freq, int32_t interleaved,
                        const int64_t* slot_mapping, int64_t num_tokens, uint16_t* q_out,
                        uint16_t* k_cache, uint16_t* v_cache, int64_t num_blocks,
                        int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0) return fail(PAGEDKV_ERR_SHAPE, "num_tokens must be >= 0");
  if (num_blocks <= 0 || block_size <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return fail(PAGEDKV_ERR_SHAPE, "sizes must be > 0");
  if (head_dim % 8 || head_dim > 512)
    return fail(PAGEDKV_ERR_UNSUPPORTED, "head_dim (%d) must be a multiple of 8, at most 512",
                head_dim);
  if (interleaved != 0 && interleaved != 1)
    return fail(PAGEDKV_ERR_SHAPE, "interleaved must be 0 or 1");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if ((int64_t)num_q_heads * head_dim > INT32_MAX || row > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE, "rows too long");
  if (num_blocks > INT64_MAX / block_size / row)
    return fail(PAGEDKV_ERR_SHAPE, "pool size overflows");
  if (num_tokens == 0) return PAGEDKV_OK;
  if (!q || !k || !v || !positions || !inv_freq || !slot_mapping || !q_out || !k_cache ||
      !v_cache)
    return fail(PAGEDKV_ERR_NULL, "every array argument must be non-NULL");
  if (!aligned(v, 16) || !aligned(v_cache, 16) || !aligned(q, 2) || !aligned(k, 2) ||
      !aligned(q_out, 2) || !aligned(k_cache, 2) || !aligned(positions, 4) ||
      !aligned(inv_freq, 4) || !aligned(slot_mapping, 8))
    return fail(PAGEDKV_ERR_ALIGN, "v and v_cache need 16-byte alignment");
  RopeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.inv_freq = inv_freq;
  a.slot_mapping = slot_mapping;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * block_size;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.interleaved = interleaved;
  const int st = check_slots(slot_mapping, num_tokens, num_blocks * block_size, stream);
  if (st) return st;
  hipError_t e = launch_kv_write_rope(a, stream);
  if (e != hipSuccess) return hip_fail(e, "rope + kv_write launch");
  return PAGEDKV_OK;
}

size_t paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t partition_tokens) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return 0;
  const int32_t sub = block_size % kKernelBlock == 0 ? block_size / kKernelBlock : 1;
  const int64_t n = nparts_bound((int64_t)max_blocks_per_seq * block_size, kKernelBlock,
                                 partition_tokens);
  return split_workspace_bytes(batch, num_q_heads, head_dim, n) +
         view_table_bytes(batch, max_blocks_per_seq, sub);
}

int paged_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                      int32_t partition_tokens, int32_t kernel, int32_t* num_partitions,
                      int32_t* tokens_per_partition, int32_t* chosen_kernel) {
  g_last_error.clear();
  int st = check_decode_sizes(max_blocks_per_seq, batch, num_q_heads, num_kv_heads, head_dim,
                              block_size, 1);
  if (st) return st;
  if (!num_partitions || !tokens_per_partition)
    return fail(PAGEDKV_ERR_NULL, "output pointers must be non-NULL");
  int32_t sub = 1;
  st = decode_block_view(block_size, &sub);
  if (st) return st;
  if (sub > 1 && partition_tokens > 0 && partition_tokens % block_size)
    return fail(PAGEDKV_ERR_SHAPE, "partition_tokens %d is not a multiple of block_size %d",
                partition_tokens, block_size);
  const int32_t mb16 = max_blocks_per_seq * sub;
  int chosen = 0;
  st = select_kernel(kernel, head_dim, num_q_heads / num_kv_heads, kKernelBlock,
                     (int64_t)mb16 * kKernelBlock, &chosen);
  if (st) return st;
  int cus = 0;
  st = cu_count(&cus);
  if (st) return st;
  DecodePlan dp{};
  st = plan_decode(kernel, chosen, batch, num_q_heads, num_kv_heads, mb16, partition_tokens, cus,
                   &dp);
  if (st) return st;
  *num_partitions = dp.plan.nparts;
  *tokens_per_partition = dp.plan.part_tokens;
  if (chosen_kernel) *chosen_kernel = dp.kernel;
  return PAGEDKV_OK;
}

int paged_decode_attention_ex(const uint16_t* q, const uint16_t* k_cache,
                              const uint16_t* v_cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                              void* workspace, size_t workspace_bytes,
                              int32_t partition_tokens, int32_t kernel, hipEvent_t ev_begin,
                              hipEvent_t ev_end, hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     kv_dtype, out, out_dtype, workspace, workspace_bytes, partition_tokens,
                     kernel, ev_begin, ev_end, stream, nullptr);
}

int paged_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, float scale, int32_t kv_dtype, void* out,
                      int32_t out_dtype, void* workspace, size_t workspace_bytes,
                      int32_t partition_tokens, int32_t kernel, hipEvent_t ev_begin,
                      hipEvent_t ev_end, hipStream_t stream) {
  const StepWrite sw{k_new, v_new, slot_mapping, k_cache, v_cache, nullptr, nullptr, 0, nullptr};
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     kv_dtype, out, out_dtype, workspace, workspace_bytes, partition_tokens,
                     kernel, ev_begin, ev_end, stream, &sw);
}

int paged_decode_step_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              const int64_t* slot_mapping, uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, float scale, int32_t kv_dtype, void* out,
                              int32_t out_dtype, int32_t partition_tokens, int32_t kernel,
                              hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  const StepWrite sw{k_new, v_new, slot_mapping, k_cache, v_cache, nullptr, nullptr, 0, nullptr};
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     kv_dtype, out, out_dtype, nullptr, 0, partition_tokens, kernel, ev_begin,
                     ev_end, stream, &sw, /*static_scratch=*/true);
}

int paged_decode_step_rope(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* positions, const float* inv_freq, int32_t interleaved,
                           const int64_t* slot_mapping, uint16_t* q_out, uint16_t* k_cache,
                           uint16_t* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                           void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                           int32_t kernel, hipEvent_t ev_begin, hipEvent_t ev_end,
                           hipStream_t stream) {
  if (!positions) {
    g_last_error.clear();
    return fail(PAGEDKV_ERR_NULL, "positions must be non-NULL");
  }
  const StepWrite sw{k_new,     v_new,    slot_mapping, k_cache, v_cache,
                     positions, inv_freq, interleaved,  q_out};
  return decode_impl(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     kv_dtype, out, out_dtype, workspace, workspace_bytes, partition_tokens,
                     kernel, ev_begin, ev_end, stream, &sw);
}

int paged_decode_attention(const uint16_t* q, const uint16_t* k_cache,
                           const uint16_t* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           float scale, float* out, void* workspace, size_t workspace_bytes,
                           int32_t partition_tokens, hipStream_t stream) {
  return paged_decode_attention_ex(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                   context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                   block_size, num_blocks, scale, PAGEDKV_DTYPE_BF16, out,
                                   PAGEDKV_DTYPE_F32, workspace, workspace_bytes,
                                   partition_tokens, PAGEDKV_KERNEL_AUTO, nullptr, nullptr,
                                   stream);
}

int paged_decode_attention_typed(const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t partition_tokens, hipStream_t stream) {
  return paged_decode_attention_ex(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                   context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                   block_size, num_blocks, scale, kv_dtype, out, out_dtype,
                                   workspace, workspace_bytes, partition_tokens,
                                   PAGEDKV_KERNEL_AUTO, nullptr, nullptr, stream);
}

int paged_prefill_attention_split(const uint16_t* q, const int32_t* cu_seqlens_q,
                                  int64_t num_tokens, int32_t max_q_len,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, float scale,
                                  int32_t kv_dtype, void* out, int32_t out_dtype,
                                  int32_t row_blocks, void* workspace, size_t workspace_bytes,
                                  int32_t partition_tokens, hipStream_t stream) {
  g_last_error.clear();
  int st = check_formats(kv_dtype, out_dtype);
  if (st) return st;
  st = check_prefill_knobs(row_blocks, partition_tokens);
  if (st) return st;
  st = check_decode_sizes(max_blocks_per_seq, batch, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks);
  if (st) return st;
  if (num_tokens < 0 || max_q_len < 0)
    return fail(PAGEDKV_ERR_SHAPE, "num_tokens and max_q_len must be >= 0");
  if (num_tokens > INT32_MAX) return fail(PAGEDKV_ERR_SHAPE, "num_tokens exceeds int32");
  const int G = num_q_heads / num_kv_heads;
  if (!supported_prefill(head_dim, G, block_size))
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "no multi-query kernel for head_dim %d, block_size %d, group size %d", head_dim,
                block_size, G);
  if (num_blocks > (int64_t)INT32_MAX / (block_size / kKernelBlock))
    return fail(PAGEDKV_ERR_SHAPE, "num_blocks * block_size / 16 exceeds int32");
  if (batch == 0 || num_tokens == 0 || max_q_len == 0) return PAGEDKV_OK;
  if (!q || !cu_seqlens_q || !k_cache || !v_cache || !context_lens || !out ||
      (max_blocks_per_seq > 0 && !block_tables))
    return fail(PAGEDKV_ERR_NULL, "q, cu_seqlens_q, k_cache, v_cache, block_tables, "
                                  "context_lens and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_seqlens_q, 4))
    return fail(PAGEDKV_ERR_ALIGN, "q, k_cache, v_cache and out need 16-byte alignment");
  int cus = 0;
  st = cu_count(&cus);
  if (st) return st;
  PrefillPlan plan{};
  st = make_prefill_plan(num_tokens, max_q_len, batch, num_q_heads, num_kv_heads, head_dim, G,
                         max_blocks_per_seq, block_size, row_blocks, partition_tokens, cus,
                         &plan);
  if (st) return st;
  PrefillArgs a{};
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.max_blocks = max_blocks_per_seq;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * kLog2eHost;
  a.ntiles = (int32_t)plan.ntiles;
  a.nb = plan.nb;
  a.kv_dtype = kv_dtype;
  a.out_dtype = out_dtype;
  a.nparts = plan.nparts;
  a.part_keys = plan.part_keys;
  if (plan.nparts > 1) {
    const size_t need = split_workspace_bytes(num_tokens, num_q_heads, head_dim, plan.nparts);
    if (!workspace || workspace_bytes < need)
      return fail(PAGEDKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(PAGEDKV_ERR_ALIGN, "workspace needs 16-byte alignment");
    char* base = static_cast<char*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(base);
    a.ws_ml = reinterpret_cast<float*>(
        base + acc_bytes(num_tokens, num_q_heads, head_dim, plan.nparts));
  }
  st = check_tables(block_tables, context_lens, batch, max_blocks_per_seq, block_size,
                    num_blocks, stream);
  if (st) return st;
  st = check_queries(cu_seqlens_q, context_lens, batch, max_blocks_per_seq, block_size,
                     num_tokens, max_q_len, stream);
  if (st) return st;
  hipError_t e = launch_prefill_mfma(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  if (plan.nparts > 1) {
    // The merge of the decode path, with the query tokens as the batch (its rows are (token,
    // query head), the layout of out and of the partials), in the form that skips rows written
    // out directly and partitions without keys.
    DecodeArgs m{};
    m.out = out;
    m.ws_acc = a.ws_acc;
    m.ws_ml = a.ws_ml;
    m.batch = (int32_t)num_tokens;
    m.num_q_heads = num_q_heads;
    m.num_kv_heads = num_kv_heads;
    m.head_dim = head_dim;
    m.block_size = block_size;
    m.nparts = plan.nparts;
    m.kv_dtype = kv_dtype;
    m.out_dtype = out_dtype;
    e = launch_prefill_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "partition merge launch");
  }
  return PAGEDKV_OK;
}

int paged_prefill_attention_ex(const uint16_t* q, const int32_t* cu_seqlens_q,
                               int64_t num_tokens, int32_t max_q_len, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               float scale, int32_t kv_dtype, void* out, int32_t out_dtype,
                               int32_t row_blocks, hipStream_t stream) {
  return paged_prefill_attention_split(q, cu_seqlens_q, num_tokens, max_q_len, k_cache, v_cache,
                                       block_tables, max_blocks_per_seq, context_lens, batch,
                                       num_q_heads, num_kv_heads, head_dim, block_size,
                                       num_blocks, scale, kv_dtype, out, out_dtype, row_blocks,
                                       nullptr, 0, -1, stream);
}

size_t paged_prefill_workspace_bytes(int64_t num_tokens, int32_t num_q_heads, int32_t head_dim,
                                     int32_t max_blocks_per_seq, int32_t block_size,
                                     int32_t partition_tokens) {
  if (num_tokens <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return 0;
  const int64_t n =
      prefill_nparts_bound((int64_t)max_blocks_per_seq * block_size, partition_tokens);
  return split_workspace_bytes(num_tokens, num_q_heads, head_dim, n);
}

int paged_prefill_plan(int64_t num_tokens, int32_t max_q_len, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t row_blocks,
                       int32_t partition_tokens, int32_t* row_blocks_used,
                       int32_t* num_partitions, int32_t* keys_per_partition) {
  g_last_error.clear();
  if (!row_blocks_used || !num_partitions || !keys_per_partition)
    return fail(PAGEDKV_ERR_NULL, "output pointers must be non-NULL");
  int st = check_decode_sizes(max_blocks_per_seq, batch, num_q_heads, num_kv_heads, head_dim,
                              block_size, 1);
  if (st) return st;
  if (num_tokens < 0 || max_q_len < 0 || num_tokens > INT32_MAX)
    return fail(PAGEDKV_ERR_SHAPE, "num_tokens and max_q_len must be in [0, 2^31)");
  const int G = num_q_heads / num_kv_heads;
  if (!supported_prefill(head_dim, G, block_size))
    return fail(PAGEDKV_ERR_UNSUPPORTED,
                "no multi-query kernel for head_dim %d, block_size %d, group size %d", head_dim,
                block_size, G);
  int cus = 0;
  st = cu_count(&cus);
  if (st) return st;
  PrefillPlan plan{};
  st = make_prefill_plan(num_tokens, max_q_len, batch, num_q_heads, num_kv_heads, head_dim, G,
                         max_blocks_per_seq, block_size, row_blocks, partition_tokens, cus,
                         &plan);
  if (st) return st;
  *row_blocks_used = plan.nb;
  *num_partitions = plan.nparts;
  *keys_per_partition = plan.part_keys;
  return PAGEDKV_OK;
}

int paged_prefill_attention(const uint16_t* q, const int32_t* cu_seqlens_q, int64_t num_tokens,
                            int32_t max_q_len, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, float scale, float* out, hipStream_t stream) {
  return paged_prefill_attention_ex(q, cu_seqlens_q, num_tokens, max_q_len, k_cache, v_cache,
                                    block_tables, max_blocks_per_seq, context_lens, batch,
                                    num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                    scale, PAGEDKV_DTYPE_BF16, out, PAGEDKV_DTYPE_F32, 0, stream);
}

}  // extern "C"
