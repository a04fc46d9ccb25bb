// Internal interface between the C ABI (rc_host.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rc {

// Plain copy of a ring's geometry and device pointers, as the kernels see it.
struct RingView {
  int N, H, d, kv, v_ld;
  float rope_base;
  int n_anchor;  // slots 0..n_anchor-1 are pinned
  int n_memory;  // slots N-n_memory..N-1 are the content memory; writes wrap from
                 // E = N - n_memory to n_anchor
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  int32_t* slot_pos;
  int32_t* slot_block;
};

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

hipError_t launch_ring_clear(const RingView& r, hipStream_t s);

// Writes n_new tokens to slots head + i, wrapping from E to n_anchor
// (n_new <= E - n_anchor).
hipError_t launch_cache_write(const RingView& r, const void* k_new, const void* v_new, int n_new,
                              int head, int pos0, int block_id, hipStream_t s);

hipError_t launch_rerotate(const RingView& r, int delta, hipStream_t s);

struct AttnCall {
  const void* q;
  int n_q, q_pos0, q_block0, q_block_len;
  float cache_bias, softmax_scale;
  void* out;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  const int32_t* q_block_ids = nullptr;  // [n_q] or null (q_block0 + i / q_block_len)
  int same_block = 0;                    // 1: visible iff slot block == query block
  int precision = 0;                     // FP8 rings: 1 two-term Q and P, 2 one-term (resolved on the host)
};

// Whether an attention kernel is built for this KV format and head size.
bool attention_supported(int kv, int d);
// Number of key splits the attention uses for n_q queries (1 = none).
int attention_splits(const RingView& r, int n_q);
size_t attention_workspace_bytes(const RingView& r, int n_q);
hipError_t launch_chunk_attention(const RingView& r, const AttnCall& c, hipStream_t s);
// FP8 rings (attn_fp8.hip): key splits for n_q queries and the launch.
int fp8_attention_splits(const RingView& r, int n_q);
hipError_t launch_fp8_attention(const RingView& r, const AttnCall& c, int splits, hipStream_t s);
// The FP8 attention kernel's half-tile classes (export for checking).
size_t debug_tile_classes_bytes(const RingView& r, int n_q);
hipError_t launch_debug_tile_classes(const RingView& r, int n_q, int q_block0, int q_block_len, bool same_block,
                                     float cache_bias, uint8_t* out, hipStream_t s);

// Attention mass per head and slot (memory.hip), optionally only for the
// slots of up to kMassRanges ranges [lo, hi) (ranges: lo, hi pairs on the
// host; n_ranges 0 = every slot).
constexpr int kMassRanges = 4;
bool key_mass_supported(int kv, int d);
size_t key_mass_workspace_bytes(const RingView& r, int n_q);
hipError_t launch_key_mass(const RingView& r, const AttnCall& c, const float* lse, float* mass, const int* ranges,
                           int n_ranges, hipStream_t s);

// Scored content memory (memory.hip): before a write of n_new tokens at
// `head`, keep the best of the memory's tokens and the history tokens the
// write evicts in the memory slots.
constexpr int kMaxMemoryCandidates = 4096;
size_t memory_workspace_bytes(int n_memory, int n_new);
hipError_t launch_memory_update(const RingView& r, const float* key_score, float gamma, int head, int n_new,
                                int n_candidates, void* workspace, hipStream_t s);

// Fused QKV projection (FP8) and cache write (qkv_write.hip); d = 128.
size_t qkv_workspace_bytes(int n, int C);
hipError_t launch_qkv_project_write(const RingView& r, const void* x, int n, int C, const uint8_t* w,
                                    const float* w_scale, int head, int pos0, int block_id, void* q_out,
                                    void* workspace, hipStream_t s);

// Record a failure for rc_last_error (rc_host.cpp) and return st.
int host_fail(int st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

hipError_t launch_debug_visibility(const RingView& r, int n_q, int q_block0, int q_block_len,
                                   uint8_t* mask, hipStream_t s);

}  // namespace rc
