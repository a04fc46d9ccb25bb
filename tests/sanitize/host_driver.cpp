// Host-only driver for the C ABI's argument and state checks, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU, no HIP runtime).
//
// The kernel launchers and workspace helpers of rc_kernels.h are replaced by
// stubs that count launches (and can report a HIP error), so every path of
// rc_host.cpp runs on the CPU.  The driver checks:
//   * hand-picked rejections of every entry point: a non-OK status, nothing
//     launched, the ring struct byte-for-byte unchanged;
//   * a valid call sequence (init, write, rewrite, advance, rerotate,
//     attention, key mass, scored write, fused projection write) and its
//     host-state updates;
//   * launch failures: RC_ERR_HIP and an unchanged host state;
//   * a seeded fuzz over ring fields and arguments, including int32 extremes,
//     with the same invariants for every rejected call.
// Any sanitizer report aborts the run with a non-zero status.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "rc.h"
#include "rc_kernels.h"

// ---------------------------------------------------------------- stubs
static long g_launches = 0;
static hipError_t g_launch_result = hipSuccess;

static hipError_t launched() {
  ++g_launches;
  return g_launch_result;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace rc {
hipError_t launch_ring_clear(const RingView&, hipStream_t) { return launched(); }
hipError_t launch_cache_write(const RingView&, const void*, const void*, int, int, int, int, hipStream_t) {
  return launched();
}
hipError_t launch_rerotate(const RingView&, int, hipStream_t) { return launched(); }
bool attention_supported(int kv, int d) { return !(kv == KV_F32 && d == 128); }
int attention_splits(const RingView&, int n_q) { return n_q < 64 ? 4 : 1; }
size_t attention_workspace_bytes(const RingView& r, int n_q) {
  return static_cast<size_t>(attention_splits(r, n_q)) * n_q * r.H * (r.d + 1) * 4;
}
hipError_t launch_chunk_attention(const RingView&, const AttnCall&, hipStream_t) { return launched(); }
int fp8_attention_splits(const RingView& r, int n_q) { return attention_splits(r, n_q); }
hipError_t launch_fp8_attention(const RingView&, const AttnCall&, int, hipStream_t) { return launched(); }
bool key_mass_supported(int kv, int) { return kv == KV_FP8; }
size_t key_mass_workspace_bytes(const RingView& r, int n_q) { return static_cast<size_t>(n_q) * r.H * 4 + 256; }
hipError_t launch_key_mass(const RingView&, const AttnCall&, const float*, float*, const int*, int, hipStream_t) {
  return launched();
}
size_t memory_workspace_bytes(int n_memory, int n_new) { return static_cast<size_t>(n_memory + n_new) * 16 + 256; }
hipError_t launch_memory_update(const RingView&, const float*, float, int, int, int, void*, hipStream_t) {
  return launched();
}
size_t qkv_workspace_bytes(int n, int C) { return static_cast<size_t>(n) * C + 256; }
hipError_t launch_qkv_project_write(const RingView&, const void*, int, int, const uint8_t*, const float*, int, int,
                                    int, void*, void*, hipStream_t) {
  return launched();
}
hipError_t launch_debug_visibility(const RingView&, int, int, int, uint8_t*, hipStream_t) { return launched(); }
size_t debug_tile_classes_bytes(const RingView& r, int n_q) {
  return static_cast<size_t>((n_q + 31) / 32) * ((r.N + 127) / 128) * 2;
}
hipError_t launch_debug_tile_classes(const RingView&, int, int, int, bool, float, uint8_t*, hipStream_t) {
  return launched();
}
}  // namespace rc

// ---------------------------------------------------------------- helpers
static int g_fail = 0;
static long g_checks = 0, g_rejections = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n",   \
                   __FILE__, __LINE__, #cond, rc_last_error());            \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// Placeholder device buffers: real heap memory, so a host-side dereference
// would be caught by the sanitizer (the library must never touch them).
struct Buffers {
  std::vector<unsigned char> mem = std::vector<unsigned char>(1 << 16);
  void* at(size_t off) { return mem.data() + ((reinterpret_cast<uintptr_t>(mem.data()) + 255) / 256 * 256 -
                                              reinterpret_cast<uintptr_t>(mem.data())) + off; }
};
static Buffers g_buf;

static rc_ring make_ring(int N, int H, int d, int kv, int A = 0, int M = 0) {
  rc_ring r;
  std::memset(&r, 0, sizeof r);
  r.n_slots = N;
  r.n_heads = H;
  r.head_dim = d;
  r.kv_dtype = kv;
  r.rope_base = 10000.f;
  r.v_ld = rc_ring_v_ld(N);
  r.n_anchor = A;
  r.n_memory = M;
  r.k = g_buf.at(0);
  r.v = g_buf.at(4096);
  r.k_scale = static_cast<float*>(g_buf.at(8192));
  r.v_scale = static_cast<float*>(g_buf.at(12288));
  r.slot_pos = static_cast<int32_t*>(g_buf.at(16384));
  r.slot_block = static_cast<int32_t*>(g_buf.at(20480));
  return r;
}

// A call that must be rejected: non-OK, nothing launched, ring unchanged.
template <class F>
static void expect_reject(rc_ring* r, rc_status want, F call, int line) {
  rc_ring before;
  if (r) std::memcpy(&before, r, sizeof before);
  const long l0 = g_launches;
  const rc_status got = call();
  ++g_rejections;
  ++g_checks;
  if (got == RC_OK || (want != RC_OK && got != want) || g_launches != l0 ||
      (r && std::memcmp(&before, r, sizeof before) != 0)) {
    std::fprintf(stderr, "line %d: rejection failed: status %d (want %d), launches %ld, state %s (%s)\n", line,
                 got, want, g_launches - l0, r && std::memcmp(&before, r, sizeof before) ? "changed" : "same",
                 rc_last_error());
    ++g_fail;
  }
  if (std::strlen(rc_last_error()) == 0) {
    std::fprintf(stderr, "line %d: rejection without a message\n", line);
    ++g_fail;
  }
}
#define REJECT(r, want, expr) expect_reject((r), (want), [&]() { return (expr); }, __LINE__)

// ---------------------------------------------------------------- cases
static void geometry_and_init() {
  size_t out[6];
  REJECT(nullptr, RC_ERR_ARG, rc_ring_sizes(0, 1, 64, RC_BF16, out));
  REJECT(nullptr, RC_ERR_ARG, rc_ring_sizes(1 << 25, 1, 64, RC_BF16, out));
  REJECT(nullptr, RC_ERR_ARG, rc_ring_sizes(100, 0, 64, RC_BF16, out));
  REJECT(nullptr, RC_ERR_ARG, rc_ring_sizes(100, 1, 64, 9, out));
  REJECT(nullptr, RC_ERR_UNSUPPORTED, rc_ring_sizes(100, 1, 96, RC_BF16, out));
  CHECK(rc_ring_sizes(1 << 24, 4096, 128, RC_F32, out) == RC_OK);  // largest geometry: sizes do not overflow
  CHECK(out[0] == static_cast<size_t>(1 << 24) * 4096 * 128 * 4);

  rc_ring r = make_ring(1000, 4, 128, RC_FP8_E4M3);
  REJECT(nullptr, RC_ERR_ARG, rc_ring_init(nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_ring_init(&r, -1, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_ring_init(&r, 1000, nullptr));
  rc_ring bad = r;
  bad.v_ld = 1000;
  REJECT(&bad, RC_ERR_ARG, rc_ring_init(&bad, 0, nullptr));
  bad = r;
  bad.k = static_cast<char*>(r.k) + 4;
  REJECT(&bad, RC_ERR_ARG, rc_ring_init(&bad, 0, nullptr));
  bad = r;
  bad.k_scale = nullptr;
  REJECT(&bad, RC_ERR_ARG, rc_ring_init(&bad, 0, nullptr));
  bad = r;
  bad.rope_base = -1.f;
  REJECT(&bad, RC_ERR_ARG, rc_ring_init(&bad, 0, nullptr));
  bad = r;
  bad.n_anchor = 600;
  bad.n_memory = 400;
  REJECT(&bad, RC_ERR_ARG, rc_ring_init(&bad, 0, nullptr));
  CHECK(rc_ring_init(&r, 7, nullptr) == RC_OK);
  CHECK(r.head == 7 && r.n_hist == 0 && r.n_cur == 0 && r.max_block == -1 && r.pos_lo > r.pos_hi);
}

static void write_sequence() {
  rc_ring r = make_ring(1000, 4, 128, RC_FP8_E4M3);
  CHECK(rc_ring_init(&r, 990, nullptr) == RC_OK);
  void* kv = g_buf.at(24576);
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, nullptr, kv, 10, 0, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, kv, static_cast<char*>(kv) + 2, 10, 0, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, kv, kv, 0, 0, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, kv, kv, 1001, 0, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, kv, kv, 10, INT32_MAX - 5, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write(&r, kv, kv, 10, 0, -1, nullptr));
  CHECK(rc_cache_write(&r, kv, kv, 20, 100, 3, nullptr) == RC_OK);  // wraps at 1000
  CHECK(r.n_cur == 20 && r.cur_pos0 == 100 && r.cur_block == 3 && r.max_block == 3);
  CHECK(r.pos_lo == 100 && r.pos_hi == 119);
  REJECT(&r, RC_ERR_STATE, rc_cache_write(&r, kv, kv, 20, 101, 3, nullptr));
  REJECT(&r, RC_ERR_STATE, rc_ring_advance(&r, 19));
  CHECK(rc_cache_write(&r, kv, kv, 20, 100, 3, nullptr) == RC_OK);  // a second denoising pass
  CHECK(rc_ring_advance(&r, 20) == RC_OK);
  CHECK(r.head == 10 && r.n_hist == 20 && r.n_cur == 0);
  // rerotate keeps every cached position inside int32 with no chunk current
  REJECT(&r, RC_ERR_ARG, rc_cache_rerotate(&r, INT32_MAX - 110, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_rerotate(&r, INT32_MAX - 119 + 1, nullptr));
  CHECK(rc_cache_rerotate(&r, INT32_MIN, nullptr) == RC_OK);  // 100 - 2^31 still fits
  CHECK(r.pos_lo == 100 + INT32_MIN && r.pos_hi == 119 + INT32_MIN);
  REJECT(&r, RC_ERR_ARG, rc_cache_rerotate(&r, -101, nullptr));
  CHECK(rc_cache_rerotate(&r, INT32_MAX, nullptr) == RC_OK);
  CHECK(rc_cache_rerotate(&r, 1 - 100, nullptr) == RC_OK);
  CHECK(r.pos_lo == 0 && r.pos_hi == 19);
  rc_ring nor = r;
  nor.rope_base = 0.f;
  REJECT(&nor, RC_ERR_ARG, rc_cache_rerotate(&nor, 5, nullptr));
  // launch failures leave the state
  g_launch_result = hipErrorInvalidValue;
  rc_ring before = r;
  CHECK(rc_cache_write(&r, kv, kv, 5, 500, 4, nullptr) == RC_ERR_HIP);
  CHECK(std::memcmp(&before, &r, sizeof r) == 0);
  CHECK(rc_cache_rerotate(&r, 1, nullptr) == RC_ERR_HIP);
  CHECK(std::memcmp(&before, &r, sizeof r) == 0);
  g_launch_result = hipSuccess;
  // corrupt host state is refused by every state-reading call
  rc_ring bad = r;
  bad.head = 5000;
  REJECT(&bad, RC_ERR_STATE, rc_cache_write(&bad, kv, kv, 5, 500, 4, nullptr));
  REJECT(&bad, RC_ERR_STATE, rc_cache_rerotate(&bad, 1, nullptr));
  REJECT(&bad, RC_ERR_STATE, rc_ring_advance(&bad, 5));
  bad = r;
  bad.n_hist = 999;
  bad.n_cur = 5;
  REJECT(&bad, RC_ERR_STATE, rc_ring_advance(&bad, 5));
}

static void attention_and_mass() {
  rc_ring r = make_ring(1000, 4, 128, RC_FP8_E4M3);
  CHECK(rc_ring_init(&r, 0, nullptr) == RC_OK);
  void* q = g_buf.at(24576);
  void* out = g_buf.at(28672);
  float* lse = static_cast<float*>(g_buf.at(32768));
  void* ws = g_buf.at(36864);
  REJECT(&r, RC_ERR_ARG, rc_chunk_attention(&r, nullptr, 10, 0, 0, 10, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_chunk_attention(&r, q, 0, 0, 0, 10, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_chunk_attention(&r, q, 10, 0, 0, 0, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG,
         rc_chunk_attention(&r, static_cast<char*>(q) + 8, 10, 0, 0, 10, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_chunk_attention_ex(&r, q, 10, 0, nullptr, 0, 10, 7, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(&r, RC_ERR_ARG,
         rc_chunk_attention_ex(&r, q, 10, 0, reinterpret_cast<const int32_t*>(static_cast<char*>(q) + 2), 0, 10, 0,
                               0.f, 0.f, out, lse, nullptr, 0, nullptr));
  REJECT(nullptr, RC_ERR_ARG, rc_set_attention_precision(3));
  CHECK(rc_attention_workspace_bytes(nullptr, 10) == 0);
  CHECK(rc_attention_workspace_bytes(&r, 0) == 0);
  rc_ring f32r = make_ring(1000, 4, 128, RC_F32);
  CHECK(rc_ring_init(&f32r, 0, nullptr) == RC_OK);
  REJECT(&f32r, RC_ERR_UNSUPPORTED, rc_chunk_attention(&f32r, q, 10, 0, 0, 10, 0.f, 0.f, out, lse, nullptr, 0, nullptr));
  // key mass
  const size_t need = rc_key_mass_workspace_bytes(&r, 10);
  float* mass = static_cast<float*>(g_buf.at(40960));
  REJECT(&r, RC_ERR_ARG, rc_key_mass(&r, q, 10, 0, 0, 10, 0.f, 0.f, nullptr, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass(&r, q, 10, INT32_MAX, 0, 10, 0.f, 0.f, lse, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass(&r, q, 10, 0, 0, 10, NAN, 0.f, lse, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass(&r, q, 10, 0, 0, 10, 0.f, -1.f, lse, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass(&r, q, 10, 0, 0, 10, 0.f, 0.f, lse, mass, ws, need - 1, nullptr));
  const int32_t bad_ranges[4] = {0, 10, 20, 2000};
  REJECT(&r, RC_ERR_ARG,
         rc_key_mass_slots(&r, q, 10, 0, 0, 10, 0.f, 0.f, lse, bad_ranges, 2, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass_slots(&r, q, 10, 0, 0, 10, 0.f, 0.f, lse, bad_ranges, 0, mass, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_key_mass_slots(&r, q, 10, 0, 0, 10, 0.f, 0.f, lse, bad_ranges, 5, mass, ws, need, nullptr));
  const int32_t ranges[4] = {0, 10, 20, 1000};
  CHECK(rc_key_mass_slots(&r, q, 10, 0, 0, 10, 0.f, 0.f, lse, ranges, 2, mass, ws, need, nullptr) == RC_OK);
  CHECK(rc_chunk_attention(&r, q, 10, 0, 0, 10, -0.5f, 0.f, out, lse, ws, 1 << 12, nullptr) == RC_OK);
  REJECT(&r, RC_ERR_ARG, rc_debug_visibility(&r, 10, 0, 10, nullptr, nullptr));
  // tile classes: size, then each rejection
  const size_t cls_bytes = rc_debug_tile_classes_bytes(&r, 40);
  CHECK(cls_bytes == 2 * ((r.n_slots + 127) / 128) * 2);
  CHECK(rc_debug_tile_classes_bytes(&r, 0) == 0);
  uint8_t* cls = static_cast<uint8_t*>(g_buf.at(32768));
  CHECK(rc_debug_tile_classes(&r, 40, 0, 10, RC_MASK_BLOCK_CAUSAL, -0.5f, cls, cls_bytes, nullptr) == RC_OK);
  CHECK(rc_debug_tile_classes(&r, 40, 0, 10, RC_MASK_SAME_BLOCK, 0.f, cls, cls_bytes, nullptr) == RC_OK);
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 40, 0, 10, RC_MASK_BLOCK_CAUSAL, 0.f, nullptr, cls_bytes, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 40, 0, 10, RC_MASK_BLOCK_CAUSAL, 0.f, cls, cls_bytes - 1, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 0, 0, 10, RC_MASK_BLOCK_CAUSAL, 0.f, cls, cls_bytes, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 40, 0, 0, RC_MASK_BLOCK_CAUSAL, 0.f, cls, cls_bytes, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 40, 0, 10, 7, 0.f, cls, cls_bytes, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_debug_tile_classes(&r, 40, 0, 10, RC_MASK_BLOCK_CAUSAL, NAN, cls, cls_bytes, nullptr));
}

static void scored_and_projection() {
  rc_ring r = make_ring(1000, 4, 128, RC_FP8_E4M3, 0, 100);
  CHECK(rc_ring_init(&r, 0, nullptr) == RC_OK);
  void* kv = g_buf.at(24576);
  float* score = static_cast<float*>(g_buf.at(45056));
  void* ws = g_buf.at(49152);
  const size_t need = rc_cache_write_scored_workspace_bytes(&r, 300);
  for (int c = 0; c < 4; ++c) {
    CHECK(rc_cache_write_scored(&r, kv, kv, 300, 300 * c, c, score, 0.5f, ws, need, nullptr) == RC_OK);
    CHECK(rc_ring_advance(&r, 300) == RC_OK);
  }
  CHECK(r.n_mem == 100 && r.n_hist == 900);
  REJECT(&r, RC_ERR_ARG, rc_cache_write_scored(&r, kv, kv, 300, 1200, 4, score, 0.f, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write_scored(&r, kv, kv, 300, 1200, 4, nullptr, 0.5f, ws, need, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write_scored(&r, kv, kv, 300, 1200, 4, score, 0.5f, ws, need - 1, nullptr));
  REJECT(&r, RC_ERR_ARG, rc_cache_write_scored(&r, kv, kv, 300, 1200, 4, score, 0.5f,
                                               static_cast<char*>(ws) + 8, need, nullptr));
  // fused projection
  rc_ring p = make_ring(1000, 4, 128, RC_FP8_E4M3);
  CHECK(rc_ring_init(&p, 0, nullptr) == RC_OK);
  const uint8_t* w = static_cast<const uint8_t*>(g_buf.at(53248));
  const float* wsc = static_cast<const float*>(g_buf.at(57344));
  void* qo = g_buf.at(61440 - 4096);
  const size_t qneed = rc_qkv_workspace_bytes(16, 512);
  REJECT(&p, RC_ERR_ARG, rc_qkv_project_write(&p, kv, 16, 500, w, wsc, 0, 0, qo, ws, qneed, nullptr));
  REJECT(&p, RC_ERR_ARG, rc_qkv_project_write(&p, kv, 16, 512, nullptr, wsc, 0, 0, qo, ws, qneed, nullptr));
  REJECT(&p, RC_ERR_ARG, rc_qkv_project_write(&p, kv, 16, 512, w, wsc, 0, 0, qo, ws, qneed - 1, nullptr));
  rc_ring p64 = make_ring(1000, 4, 64, RC_FP8_E4M3);
  CHECK(rc_ring_init(&p64, 0, nullptr) == RC_OK);
  REJECT(&p64, RC_ERR_UNSUPPORTED, rc_qkv_project_write(&p64, kv, 16, 512, w, wsc, 0, 0, qo, ws, qneed, nullptr));
  CHECK(rc_qkv_project_write(&p, kv, 16, 512, w, wsc, INT32_MAX - 15, 2, qo, ws, qneed, nullptr) == RC_OK);
  CHECK(p.pos_hi == INT32_MAX && p.pos_lo == INT32_MAX - 15);
  REJECT(&p, RC_ERR_ARG, rc_cache_rerotate(&p, 1, nullptr));
}

// Seeded fuzz: random (often invalid) rings and arguments.  Every call must
// either succeed or be a clean rejection.
static void fuzz(int iters) {
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<long long> v) { return *(v.begin() + rng() % v.size()); };
  auto rint = [&]() -> int32_t {
    return static_cast<int32_t>(pick({0, 1, -1, 2, 7, 63, 64, 100, 757, 1000, 5788, INT32_MAX, INT32_MIN,
                                      INT32_MAX - 1, INT32_MIN + 1, static_cast<long long>(rng() % 20000) - 5000}));
  };
  void* kv = g_buf.at(24576);
  void* out = g_buf.at(28672);
  float* lse = static_cast<float*>(g_buf.at(32768));
  void* ws = g_buf.at(36864);
  for (int it = 0; it < iters; ++it) {
    rc_ring r = make_ring(static_cast<int>(pick({1, 2, 100, 1000, 5788, 0, -3, 1 << 25})),
                          static_cast<int>(pick({1, 4, 40, 0, 5000})), static_cast<int>(pick({64, 128, 96})),
                          static_cast<int>(pick({0, 1, 2, 3})), static_cast<int>(pick({0, 0, 1, 30, 99})),
                          static_cast<int>(pick({0, 0, 1, 20, 500})));
    if (rng() % 4 == 0) r.v_ld = rint();
    if (rng() % 3 == 0) {
      r.head = rint();
      r.n_hist = rint();
      r.n_cur = rint();
      r.cur_pos0 = rint();
      r.cur_block = rint();
      r.n_mem = rint();
      r.max_block = rint();
      r.pos_lo = rint();
      r.pos_hi = rint();
    } else if (rc_ring_init(&r, static_cast<int32_t>(rng() % 8), nullptr) != RC_OK) {
      continue;
    }
    rc_ring before = r;
    const long l0 = g_launches;
    rc_status st;
    const int which = static_cast<int>(rng() % 6);
    switch (which) {
      case 0: st = rc_cache_write(&r, kv, kv, rint(), rint(), rint(), nullptr); break;
      case 1: st = rc_cache_rerotate(&r, rint(), nullptr); break;
      case 2: st = rc_ring_advance(&r, rint()); break;
      case 3:
        st = rc_chunk_attention(&r, kv, rint(), rint(), rint(), rint(), 0.f, 0.f, out, lse, ws, 4096, nullptr);
        break;
      case 4: {
        const size_t need = rc_key_mass_workspace_bytes(&r, 10);
        st = rc_key_mass(&r, kv, rint(), rint(), rint(), rint(), -1.f, 0.f, lse, lse, ws, need, nullptr);
        break;
      }
      default: {
        const size_t need = rc_cache_write_scored_workspace_bytes(&r, 10);
        st = rc_cache_write_scored(&r, kv, kv, rint(), rint(), rint(), lse, 0.5f, ws, need, nullptr);
      }
    }
    if (st != RC_OK) {
      ++g_rejections;
      CHECK(g_launches == l0);
      CHECK(std::memcmp(&before, &r, sizeof r) == 0);
    } else if (which != 4 && which != 2) {
      // every call but the key mass and the advance (which checks only the
      // ring's slot counts) validates the ring and its host state, and an
      // accepted call leaves both consistent: a call that checks them accepts
      const int32_t n_cur = r.n_cur;
      if (n_cur > 0) CHECK(rc_ring_advance(&r, n_cur) == RC_OK);
      else CHECK(rc_cache_rerotate(&r, 0, nullptr) == RC_OK);
    }
  }
}

int main() {
  geometry_and_init();
  write_sequence();
  attention_and_mass();
  scored_and_projection();
  fuzz(200000);
  std::printf("host driver: %ld checks, %ld rejections, %ld stub launches, %d failures\n", g_checks, g_rejections,
              g_launches, g_fail);
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
