// A native caller of the C ABI (include/paged_kv.h), with no Python in the way: it builds a
// small paged cache on the device, runs the fused decode step eagerly, records several steps
// into a HIP graph with the runtime's stream capture (as a serving loop records every layer's
// step), replays the graph, and checks:
//   - every replay leaves the output and both pools bit-identical to the eager step;
//   - the fused step equals paged_kv_write followed by paged_decode_attention_ex, bit for bit;
//   - a sequence of length 1 returns its new value row exactly (one weight of exactly 1);
//   - the checked build's status call answers as its build says.
// Exit status 0 on success; the first failed check is printed. Built by the package's build
// step (next to the library); run by tests/test_native_abi.py.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "paged_kv.h"

namespace {

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    const hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,                \
                   hipGetErrorString(e_));                                          \
      return 2;                                                                     \
    }                                                                               \
  } while (0)

#define LIB_OK(x)                                                                   \
  do {                                                                              \
    const int s_ = (x);                                                             \
    if (s_ != PAGEDKV_OK) {                                                         \
      std::fprintf(stderr, "%s:%d %s: %s (%s)\n", __FILE__, __LINE__, #x,           \
                   paged_kv_status_string(s_), paged_kv_last_error());              \
      return 3;                                                                     \
    }                                                                               \
  } while (0)

#define CHECK(cond, msg)                                                            \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "check failed: %s\n", msg);                              \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

// A deterministic stream of bf16 values from a 64-bit linear congruential generator: the
// upper bits give a float in [-2, 2), rounded to bf16 by truncation (any bf16 values do here).
struct Gen {
  uint64_t s;
  uint16_t bf16() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    const float f = (float)((s >> 40) & 0xffffff) / (float)(1 << 22) - 2.0f;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
};

template <class T>
int upload(T** dev, const std::vector<T>& host) {
  HIP_OK(hipMalloc(reinterpret_cast<void**>(dev), host.size() * sizeof(T)));
  HIP_OK(hipMemcpy(*dev, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice));
  return 0;
}

template <class T>
int download(std::vector<T>& host, const T* dev) {
  HIP_OK(hipMemcpy(host.data(), dev, host.size() * sizeof(T), hipMemcpyDeviceToHost));
  return 0;
}

int run() {
  // 4 sequences (lengths 1, 300, 1200, 2100) over a 544-block pool of 16-token blocks,
  // 8 query / 2 KV heads, head_dim 128, bf16 in, fp32 out.
  const int B = 4, Hq = 8, Hkv = 2, D = 128, bs = 16, NB = 544, MB = 160;
  const int lens[B] = {1, 300, 1200, 2100};
  const float scale = 1.0f / std::sqrt((float)D);
  const size_t row = (size_t)Hkv * D;
  Gen g{12345};

  // Block tables: sequence b takes blocks b, b + 4, b + 8, ... (disjoint, scattered); -1 past
  // its context. The new token's slot is the table's slot of position L - 1.
  std::vector<int32_t> tables((size_t)B * MB, -1);
  std::vector<int64_t> slots(B);
  for (int b = 0; b < B; ++b) {
    const int nblk = (lens[b] + bs - 1) / bs;
    for (int j = 0; j < nblk; ++j) tables[(size_t)b * MB + j] = b + 4 * j;
    const int p = lens[b] - 1;
    slots[b] = (int64_t)tables[(size_t)b * MB + p / bs] * bs + p % bs;
  }
  std::vector<uint16_t> kc((size_t)NB * bs * row), vc(kc.size());
  for (auto& x : kc) x = g.bf16();
  for (auto& x : vc) x = g.bf16();
  std::vector<uint16_t> q((size_t)B * Hq * D), kn((size_t)B * row), vn(kn.size());
  for (auto& x : q) x = g.bf16();
  for (auto& x : kn) x = g.bf16();
  for (auto& x : vn) x = g.bf16();
  std::vector<int32_t> lv(lens, lens + B);

  int32_t *d_tables, *d_lens;
  int64_t* d_slots;
  uint16_t *d_q, *d_kn, *d_vn, *d_kc, *d_vc, *d_kc2, *d_vc2;
  if (upload(&d_tables, tables) || upload(&d_lens, lv) || upload(&d_slots, slots) ||
      upload(&d_q, q) || upload(&d_kn, kn) || upload(&d_vn, vn) || upload(&d_kc, kc) ||
      upload(&d_vc, vc) || upload(&d_kc2, kc) || upload(&d_vc2, vc))
    return 2;
  float *d_out, *d_ref;
  HIP_OK(hipMalloc(&d_out, (size_t)B * Hq * D * 4));
  HIP_OK(hipMalloc(&d_ref, (size_t)B * Hq * D * 4));
  const size_t ws_bytes = paged_decode_workspace_bytes(B, Hq, D, MB, bs, 0);
  void* d_ws = nullptr;
  if (ws_bytes) HIP_OK(hipMalloc(&d_ws, ws_bytes));
  hipStream_t st;
  HIP_OK(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));

  const auto step = [&](float* out, uint16_t* k_cache, uint16_t* v_cache) {
    return paged_decode_step(d_q, d_kn, d_vn, d_slots, k_cache, v_cache, d_tables, MB, d_lens, B,
                             Hq, Hkv, D, bs, NB, scale, PAGEDKV_DTYPE_BF16, out,
                             PAGEDKV_DTYPE_F32, d_ws, ws_bytes, 0, PAGEDKV_KERNEL_AUTO, nullptr,
                             nullptr, st);
  };

  // Eager fused step.
  LIB_OK(step(d_out, d_kc, d_vc));
  HIP_OK(hipStreamSynchronize(st));
  std::vector<float> eager((size_t)B * Hq * D), got(eager.size());
  std::vector<uint16_t> kc_eager(kc.size()), vc_eager(vc.size()), pool(kc.size());
  if (download(eager, d_out) || download(kc_eager, d_kc) || download(vc_eager, d_vc)) return 2;

  // The separate calls on a second copy of the pools: the same bits.
  LIB_OK(paged_kv_write(d_kn, d_vn, d_slots, B, d_kc2, d_vc2, NB, bs, Hkv, D, st));
  LIB_OK(paged_decode_attention_ex(d_q, d_kc2, d_vc2, d_tables, MB, d_lens, B, Hq, Hkv, D, bs, NB,
                                   scale, PAGEDKV_DTYPE_BF16, d_ref, PAGEDKV_DTYPE_F32, d_ws,
                                   ws_bytes, 0, PAGEDKV_KERNEL_AUTO, nullptr, nullptr, st));
  HIP_OK(hipStreamSynchronize(st));
  if (download(got, d_ref)) return 2;
  CHECK(std::memcmp(got.data(), eager.data(), got.size() * 4) == 0,
        "fused step differs from write + attention");
  if (download(pool, d_kc2)) return 2;
  CHECK(pool == kc_eager, "key pool differs between the fused step and the separate write");

  // Sequence 0 has one token: its output is its new value row, exactly.
  for (int h = 0; h < Hq; ++h) {
    const int gk = h / (Hq / Hkv);
    for (int d = 0; d < D; ++d) {
      const uint32_t u = (uint32_t)vn[(size_t)gk * D + d] << 16;
      float v;
      std::memcpy(&v, &u, 4);
      CHECK(eager[(size_t)h * D + d] == v, "a one-token context does not return its value row");
    }
  }

  // Eight steps recorded into one graph by the runtime's stream capture, replayed three times.
  hipGraph_t graph;
  hipGraphExec_t exec;
  HIP_OK(hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed));
  for (int i = 0; i < 8; ++i) LIB_OK(step(d_out, d_kc, d_vc));
  HIP_OK(hipStreamEndCapture(st, &graph));
  HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  for (int r = 0; r < 3; ++r) {
    HIP_OK(hipMemsetAsync(d_out, 0xff, (size_t)B * Hq * D * 4, st));  // NaN, outside the graph
    HIP_OK(hipGraphLaunch(exec, st));
    HIP_OK(hipStreamSynchronize(st));
    if (download(got, d_out)) return 2;
    CHECK(std::memcmp(got.data(), eager.data(), got.size() * 4) == 0,
          "a graph replay differs from the eager step");
    if (download(pool, d_kc)) return 2;
    CHECK(pool == kc_eager, "a graph replay left a different key pool");
    if (download(pool, d_vc)) return 2;
    CHECK(pool == vc_eager, "a graph replay left a different value pool");
  }
  HIP_OK(hipGraphExecDestroy(exec));
  HIP_OK(hipGraphDestroy(graph));

  // The status call of the checked build (PAGEDKV_CHECKED) answers as the build says.
  int32_t code = -1;
  const int s = paged_kv_check_status(&code, nullptr, nullptr, 1);
  if (paged_kv_checked_build()) {
    CHECK(s == PAGEDKV_OK && code == PAGEDKV_CHECK_NONE, "valid inputs left a check record");
  } else {
    CHECK(s == PAGEDKV_ERR_UNSUPPORTED, "the unchecked build answered the status call");
  }

  HIP_OK(hipStreamDestroy(st));
  for (void* p : {(void*)d_tables, (void*)d_lens, (void*)d_slots, (void*)d_q, (void*)d_kn,
                  (void*)d_vn, (void*)d_kc, (void*)d_vc, (void*)d_kc2, (void*)d_vc2,
                  (void*)d_out, (void*)d_ref})
    HIP_OK(hipFree(p));
  if (d_ws) HIP_OK(hipFree(d_ws));
  std::printf("native ABI ok: fused step = write + attention, one-token row exact, 8-step "
              "graph replayed 3x bit-identical (%s build, kernel ABI %d)\n",
              paged_kv_checked_build() ? "checked" : "default", paged_kv_abi_version());
  return 0;
}

}  // namespace

int main() { return run(); }
