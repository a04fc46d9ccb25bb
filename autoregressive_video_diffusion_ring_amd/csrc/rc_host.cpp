// C ABI of the ring-cache library: argument and state checks, ring
// bookkeeping on the host, kernel launches on the caller's stream.
//
// Ring bookkeeping (Runway Characters, abstract: a ring cache written once per
// chunk): N slots, `head` the next slot to write, the n_hist committed history
// tokens just before it.  A write of n tokens covers (head + i) mod N; it
// evicts the oldest history slots it overwrites, so n_hist becomes
// min(n_hist, N - n).  The chunk stays "current" (n_cur = n) through its
// denoising passes, each of which writes the same slots again, until
// rc_ring_advance commits it: head += n (mod N), n_hist += n, n_cur = 0.
// With an anchor of A slots and a content memory of M slots the ring part
// is slots A..E-1, E = N - M: every wrap goes from E back to A, so the first
// A tokens of the stream stay in slots 0..A-1 (the anchor starts filling at
// slot 0), and a chunk holds at most E - A tokens.  n_hist counts anchor and
// ring-part tokens (at most E); a write evicts the oldest tokens of the ring
// part only.  The memory slots E..N-1 are filled only by scored writes, which
// keep them a prefix: n_mem occupied slots are E..E+n_mem-1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/rc.h"
#include "rc_kernels.h"

// The layout the Python binding mirrors.
static_assert(offsetof(rc_ring, n_anchor) == 24 && offsetof(rc_ring, n_memory) == 28, "rc_ring layout");
static_assert(offsetof(rc_ring, k) == 32 && offsetof(rc_ring, head) == 80, "rc_ring layout");
static_assert(offsetof(rc_ring, n_mem) == 100 && offsetof(rc_ring, max_block) == 104, "rc_ring layout");
static_assert(offsetof(rc_ring, pos_lo) == 108 && offsetof(rc_ring, pos_hi) == 112, "rc_ring layout");
static_assert(sizeof(rc_ring) == 120, "rc_ring layout");

namespace {

thread_local std::string g_err;
std::atomic<int> g_precision{RC_PRECISION_AUTO};

rc_status fail(rc_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rc_status fail(rc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

int rc::host_fail(int st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

namespace {

rc_status ok() {
  g_err.clear();
  return RC_OK;
}

rc_status hip_fail(hipError_t e, const char* what) {
  return fail(RC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(int32_t dt) { return dt == RC_F32 ? 4 : (dt == RC_BF16 ? 2 : 1); }

rc_status check_geometry(int32_t n_slots, int32_t n_heads, int32_t head_dim, int32_t kv_dtype) {
  if (n_slots < 1) return fail(RC_ERR_ARG, "n_slots must be >= 1 (got %d)", n_slots);
  if (n_slots > (1 << 24)) return fail(RC_ERR_ARG, "n_slots too large (%d)", n_slots);
  if (n_heads < 1 || n_heads > 4096) return fail(RC_ERR_ARG, "n_heads must be in 1..4096 (got %d)", n_heads);
  if (kv_dtype != RC_F32 && kv_dtype != RC_BF16 && kv_dtype != RC_FP8_E4M3)
    return fail(RC_ERR_ARG, "unknown kv_dtype %d", kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(RC_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  return RC_OK;
}

rc_status check_ring(const rc_ring* r) {
  if (!r) return fail(RC_ERR_ARG, "ring is NULL");
  rc_status st = check_geometry(r->n_slots, r->n_heads, r->head_dim, r->kv_dtype);
  if (st != RC_OK) return st;
  if (r->v_ld != rc_ring_v_ld(r->n_slots))
    return fail(RC_ERR_ARG, "v_ld must be rc_ring_v_ld(n_slots) = %d (got %d)", rc_ring_v_ld(r->n_slots), r->v_ld);
  if (!std::isfinite(r->rope_base) || r->rope_base < 0.f) return fail(RC_ERR_ARG, "rope_base must be >= 0");
  if (r->n_anchor < 0 || r->n_memory < 0 || static_cast<long long>(r->n_anchor) + r->n_memory >= r->n_slots)
    return fail(RC_ERR_ARG, "need n_anchor >= 0, n_memory >= 0, n_anchor + n_memory < N (got %d, %d, N %d)",
                r->n_anchor, r->n_memory, r->n_slots);
  if (!r->k || !r->v || !r->slot_pos || !r->slot_block) return fail(RC_ERR_ARG, "ring device pointer is NULL");
  if (r->kv_dtype == RC_FP8_E4M3 && (!r->k_scale || !r->v_scale))
    return fail(RC_ERR_ARG, "FP8 ring needs k_scale and v_scale");
  const uintptr_t al = reinterpret_cast<uintptr_t>(r->k) | reinterpret_cast<uintptr_t>(r->v);
  if (al & 15u) return fail(RC_ERR_ARG, "k and v must be 16-byte aligned");
  return RC_OK;
}

// End of the ring part (first memory slot).
int32_t ring_end(const rc_ring* r) { return r->n_slots - r->n_memory; }

rc_status check_state(const rc_ring* r) {
  const int E = ring_end(r);
  if (r->head < 0 || r->head >= E || r->n_hist < 0 || r->n_cur < 0 ||
      static_cast<long long>(r->n_hist) + r->n_cur > E ||
      r->n_mem < 0 || r->n_mem > r->n_memory || r->max_block < -1)
    return fail(RC_ERR_STATE, "ring host state is corrupt (head %d, n_hist %d, n_cur %d, n_mem %d, E %d)", r->head,
                r->n_hist, r->n_cur, r->n_mem, E);
  // the current chunk's positions lie inside the bound of cached positions
  if (r->n_cur > 0 && (r->cur_pos0 < r->pos_lo || static_cast<long long>(r->cur_pos0) + r->n_cur - 1 > r->pos_hi))
    return fail(RC_ERR_STATE, "ring host state is corrupt (chunk positions %d + %d outside %d..%d)", r->cur_pos0,
                r->n_cur, r->pos_lo, r->pos_hi);
  return RC_OK;
}

rc::RingView view(const rc_ring* r) {
  rc::RingView v{};
  v.N = r->n_slots;
  v.H = r->n_heads;
  v.d = r->head_dim;
  v.kv = r->kv_dtype;
  v.v_ld = r->v_ld;
  v.n_anchor = r->n_anchor;
  v.n_memory = r->n_memory;
  v.rope_base = r->rope_base;
  v.k = r->k;
  v.v = r->v;
  v.k_scale = r->k_scale;
  v.v_scale = r->v_scale;
  v.slot_pos = r->slot_pos;
  v.slot_block = r->slot_block;
  return v;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The slot n places after `head`, wrapping from the ring part's end E to its
// first slot (n_anchor); n <= E - n_anchor.
int32_t step_slot(const rc_ring* r, int32_t head, int32_t n) {
  const int32_t s = head + n;
  const int32_t E = ring_end(r);
  return s < E ? s : s - E + r->n_anchor;
}

// Argument and state checks shared by both writes.
rc_status check_write(const rc_ring* r, const void* k_new, const void* v_new, int32_t n_new, int32_t pos0,
                      int32_t block_id) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if ((st = check_state(r)) != RC_OK) return st;
  if (!k_new || !v_new) return fail(RC_ERR_ARG, "k_new / v_new is NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15u)
    return fail(RC_ERR_ARG, "k_new and v_new must be 16-byte aligned");
  const int32_t cap = ring_end(r) - r->n_anchor;
  if (n_new < 1 || n_new > cap)
    return fail(RC_ERR_ARG, "n_new must be in 1..%d (N - n_anchor - n_memory; got %d)", cap, n_new);
  if (block_id < 0) return fail(RC_ERR_ARG, "block_id must be >= 0 (got %d)", block_id);
  if (static_cast<long long>(pos0) + n_new - 1 > INT32_MAX) return fail(RC_ERR_ARG, "positions overflow int32");
  if (r->n_cur > 0 && (n_new != r->n_cur || pos0 != r->cur_pos0 || block_id != r->cur_block))
    return fail(RC_ERR_STATE,
                "chunk (n %d, pos0 %d, block %d) is current; a rewrite must repeat it (got n %d, pos0 %d, block %d)",
                r->n_cur, r->cur_pos0, r->cur_block, n_new, pos0, block_id);
  return RC_OK;
}

// Widen the bound of cached positions by a write of n tokens from pos0 (the
// caller has checked pos0 + n - 1 <= INT32_MAX).
void note_positions(rc_ring* r, int32_t pos0, int32_t n) {
  r->pos_lo = std::min(r->pos_lo, pos0);
  r->pos_hi = std::max(r->pos_hi, pos0 + (n - 1));
}

// Launch the write and update the host state.
rc_status do_write(rc_ring* r, const void* k_new, const void* v_new, int32_t n_new, int32_t pos0, int32_t block_id,
                   hipStream_t stream) {
  hipError_t e = rc::launch_cache_write(view(r), k_new, v_new, n_new, r->head, pos0, block_id, stream);
  if (e != hipSuccess) return hip_fail(e, "cache write");
  if (r->n_cur == 0) r->n_hist = std::min(r->n_hist, ring_end(r) - n_new);
  r->n_cur = n_new;
  r->cur_pos0 = pos0;
  r->cur_block = block_id;
  r->max_block = std::max(r->max_block, block_id);
  note_positions(r, pos0, n_new);
  return ok();
}

// Operand precision of one FP8 attention call (RC_PRECISION_AUTO resolved;
// see rc_set_attention_precision in rc.h).  The effective number of keys of a
// query that sees x slots of its own block (weight 1) and n - x earlier ones
// (weight w = exp(bias)) is f(x) = (x + (n - x) w)^2 / (x + (n - x) w^2); f
// falls to its minimum 4 n w / (1 + w)^2 at x* = n w / (1 + w) and rises
// after, so over the splits x >= x_lo the bound is f(max(x*, x_lo)).
constexpr double kFastMinKeys = 2048.0;

int attention_precision(const rc_ring* r, int mode, const int32_t* q_block, int32_t n_q, int32_t q_block0,
                        int32_t q_block_len, int32_t mask, float cache_bias) {
  if (mode != RC_PRECISION_AUTO) return mode;
  if (q_block || mask != RC_MASK_BLOCK_CAUSAL) return RC_PRECISION_TWO_TERM;
  if (q_block0 + (n_q - 1) / q_block_len != q_block0) return RC_PRECISION_TWO_TERM;
  if (r->max_block < 0 || q_block0 < r->max_block) return RC_PRECISION_TWO_TERM;
  const double n = static_cast<double>(r->n_hist) + r->n_cur + r->n_mem;
  const double x_lo = (q_block0 == r->cur_block && r->n_cur > 0) ? r->n_cur : 0.0;
  if (q_block0 > r->max_block || n <= 0.0) {  // no slot is in the queries' block
    const double w = std::exp(static_cast<double>(cache_bias));
    return n > 0.0 && std::isfinite(w) && w > 0.0 && n >= kFastMinKeys ? RC_PRECISION_ONE_TERM
                                                                       : RC_PRECISION_TWO_TERM;
  }
  const double w = std::exp(static_cast<double>(cache_bias));
  if (!std::isfinite(w)) return RC_PRECISION_TWO_TERM;
  const double x = std::min(n, std::max(n * w / (1.0 + w), x_lo));
  const double u = x + (n - x) * w, v = x + (n - x) * w * w;
  return v > 0.0 && u * u >= kFastMinKeys * v ? RC_PRECISION_ONE_TERM : RC_PRECISION_TWO_TERM;
}

}  // namespace

extern "C" {

int32_t rc_ring_v_ld(int32_t n_slots) {
  if (n_slots < 1) return 0;
  return (n_slots + 127) / 128 * 128;
}

rc_status rc_ring_sizes(int32_t n_slots, int32_t n_heads, int32_t head_dim, int32_t kv_dtype, size_t out[6]) {
  if (!out) return fail(RC_ERR_ARG, "out is NULL");
  rc_status st = check_geometry(n_slots, n_heads, head_dim, kv_dtype);
  if (st != RC_OK) return st;
  const size_t es = elem_size(kv_dtype);
  const size_t ld = rc_ring_v_ld(n_slots);
  out[0] = static_cast<size_t>(n_heads) * ld * head_dim * es;
  out[1] = static_cast<size_t>(n_heads) * head_dim * ld * es;
  out[2] = out[3] = kv_dtype == RC_FP8_E4M3 ? static_cast<size_t>(n_heads) * ld * sizeof(float) : 0;
  out[4] = out[5] = ld * sizeof(int32_t);
  return ok();
}

rc_status rc_ring_init(rc_ring* r, int32_t first_slot, void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if (first_slot < 0 || first_slot >= r->n_slots)
    return fail(RC_ERR_ARG, "first_slot must be in 0..%d (got %d)", r->n_slots - 1, first_slot);
  if (r->n_anchor > 0 && first_slot != 0)
    return fail(RC_ERR_ARG, "a ring with an anchor starts at slot 0 (got first_slot %d)", first_slot);
  if (first_slot >= ring_end(r))
    return fail(RC_ERR_ARG, "first_slot must lie before the memory slots (got %d, E %d)", first_slot, ring_end(r));
  hipError_t e = rc::launch_ring_clear(view(r), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "ring clear");
  r->head = first_slot;
  r->n_hist = 0;
  r->n_cur = 0;
  r->cur_pos0 = 0;
  r->cur_block = 0;
  r->n_mem = 0;
  r->max_block = -1;
  r->pos_lo = INT32_MAX;
  r->pos_hi = INT32_MIN;
  return ok();
}

rc_status rc_cache_write(rc_ring* r, const void* k_new, const void* v_new, int32_t n_new, int32_t pos0,
                         int32_t block_id, void* stream) {
  rc_status st = check_write(r, k_new, v_new, n_new, pos0, block_id);
  if (st != RC_OK) return st;
  return do_write(r, k_new, v_new, n_new, pos0, block_id, as_stream(stream));
}

size_t rc_cache_write_scored_workspace_bytes(const rc_ring* r, int32_t n_new) {
  if (check_ring(r) != RC_OK || n_new < 1) return 0;
  return rc::memory_workspace_bytes(r->n_memory, n_new);
}

rc_status rc_cache_write_scored(rc_ring* r, const void* k_new, const void* v_new, int32_t n_new, int32_t pos0,
                                int32_t block_id, const float* key_score, float diversity, void* workspace,
                                size_t workspace_bytes, void* stream) {
  rc_status st = check_write(r, k_new, v_new, n_new, pos0, block_id);
  if (st != RC_OK) return st;
  const int32_t E = ring_end(r);
  // history tokens this write overwrites (none on a rewrite of the current chunk)
  const int32_t evicted = r->n_cur == 0 ? r->n_hist - std::min(r->n_hist, E - n_new) : 0;
  const bool update = r->n_memory > 0 && evicted > 0;
  if (r->n_memory > 0 && r->n_cur == 0) {
    if (!(diversity > 0.f && diversity <= 1.f)) return fail(RC_ERR_ARG, "diversity must be in (0, 1]");
    if (!key_score) return fail(RC_ERR_ARG, "key_score is NULL");
    if (reinterpret_cast<uintptr_t>(key_score) & 3u) return fail(RC_ERR_ARG, "key_score must be 4-byte aligned");
    if (static_cast<long long>(r->n_memory) + n_new > rc::kMaxMemoryCandidates)
      return fail(RC_ERR_UNSUPPORTED, "n_memory + n_new must be <= %d (got %d + %d)", rc::kMaxMemoryCandidates,
                  r->n_memory, n_new);
    const size_t need = rc::memory_workspace_bytes(r->n_memory, n_new);
    if (!workspace || workspace_bytes < need)
      return fail(RC_ERR_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(RC_ERR_ARG, "workspace must be 16-byte aligned");
  }
  if (update) {
    hipError_t e = rc::launch_memory_update(view(r), key_score, diversity, r->head, n_new, r->n_mem + evicted,
                                            workspace, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "memory update");
  }
  st = do_write(r, k_new, v_new, n_new, pos0, block_id, as_stream(stream));
  if (st == RC_OK && update) r->n_mem = std::min(r->n_memory, r->n_mem + evicted);
  return st;
}

size_t rc_qkv_workspace_bytes(int32_t n, int32_t C) {
  if (n < 1 || C < 128 || C % 128) return 0;
  return rc::qkv_workspace_bytes(n, C);
}

rc_status rc_qkv_project_write(rc_ring* r, const void* x, int32_t n, int32_t C, const uint8_t* w,
                               const float* w_scale, int32_t pos0, int32_t block_id, void* q_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  rc_status st = check_write(r, x, x, n, pos0, block_id);
  if (st != RC_OK) return st;
  if (r->kv_dtype != RC_FP8_E4M3 || r->head_dim != 128)
    return fail(RC_ERR_UNSUPPORTED, "the fused projection is built for FP8 rings with head_dim 128");
  if (C < 128 || C % 128 || C > (1 << 16)) return fail(RC_ERR_ARG, "C must be a multiple of 128 in 128..65536 (got %d)", C);
  if (!w || !w_scale || !q_out) return fail(RC_ERR_ARG, "w / w_scale / q_out is NULL");
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(q_out)) & 15u)
    return fail(RC_ERR_ARG, "w and q_out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(w_scale) & 3u) return fail(RC_ERR_ARG, "w_scale must be 4-byte aligned");
  const size_t need = rc::qkv_workspace_bytes(n, C);
  if (!workspace || workspace_bytes < need)
    return fail(RC_ERR_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(RC_ERR_ARG, "workspace must be 16-byte aligned");
  hipError_t e = rc::launch_qkv_project_write(view(r), x, n, C, w, w_scale, r->head, pos0, block_id, q_out, workspace,
                                              as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "qkv projection write");
  if (r->n_cur == 0) r->n_hist = std::min(r->n_hist, ring_end(r) - n);
  r->n_cur = n;
  r->cur_pos0 = pos0;
  r->cur_block = block_id;
  r->max_block = std::max(r->max_block, block_id);
  note_positions(r, pos0, n);
  return ok();
}

rc_status rc_cache_rerotate(rc_ring* r, int32_t delta, void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if ((st = check_state(r)) != RC_OK) return st;
  if (!(r->rope_base > 0.f)) return fail(RC_ERR_ARG, "rerotate needs a ring with RoPE (rope_base > 0)");
  // every cached position lies in pos_lo .. pos_hi (a superset once slots
  // are evicted), whether or not a chunk is current
  const bool written = r->pos_lo <= r->pos_hi;
  if (written && (static_cast<long long>(r->pos_lo) + delta < INT32_MIN ||
                  static_cast<long long>(r->pos_hi) + delta > INT32_MAX))
    return fail(RC_ERR_ARG, "delta %d takes cached positions %d..%d outside int32", delta, r->pos_lo, r->pos_hi);
  hipError_t e = rc::launch_rerotate(view(r), delta, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "rerotate");
  if (r->n_cur > 0) r->cur_pos0 += delta;
  if (written) {
    r->pos_lo += delta;
    r->pos_hi += delta;
  }
  return ok();
}

rc_status rc_set_attention_precision(int32_t mode) {
  if (mode != RC_PRECISION_AUTO && mode != RC_PRECISION_TWO_TERM && mode != RC_PRECISION_ONE_TERM)
    return fail(RC_ERR_ARG, "unknown attention precision mode %d", mode);
  g_precision.store(mode);
  return ok();
}

size_t rc_attention_workspace_bytes(const rc_ring* r, int32_t n_q) {
  if (check_ring(r) != RC_OK || n_q < 1) return 0;
  return rc::attention_workspace_bytes(view(r), n_q);
}

rc_status rc_chunk_attention_ex(const rc_ring* r, const void* q, int32_t n_q, int32_t q_pos0, const int32_t* q_block,
                                int32_t q_block0, int32_t q_block_len, int32_t mask, float cache_bias,
                                float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if (!rc::attention_supported(r->kv_dtype, r->head_dim))
    return fail(RC_ERR_UNSUPPORTED, "no attention kernel for float32 rings with head_dim %d", r->head_dim);
  if (!q || !out) return fail(RC_ERR_ARG, "q / out is NULL");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15u)
    return fail(RC_ERR_ARG, "q and out must be 16-byte aligned");
  if (n_q < 1) return fail(RC_ERR_ARG, "n_q must be >= 1 (got %d)", n_q);
  if (!q_block && q_block_len < 1) return fail(RC_ERR_ARG, "q_block_len must be >= 1 (got %d)", q_block_len);
  if (q_block && (reinterpret_cast<uintptr_t>(q_block) & 3u)) return fail(RC_ERR_ARG, "q_block must be 4-byte aligned");
  if (mask != RC_MASK_BLOCK_CAUSAL && mask != RC_MASK_SAME_BLOCK) return fail(RC_ERR_ARG, "unknown mask %d", mask);
  if (static_cast<long long>(q_pos0) + n_q - 1 > INT32_MAX) return fail(RC_ERR_ARG, "positions overflow int32");
  if (!q_block && static_cast<long long>(q_block0) + (n_q - 1) / q_block_len > INT32_MAX)
    return fail(RC_ERR_ARG, "query blocks overflow int32");
  // the FP8 operand precision reads the host state
  if ((st = check_state(r)) != RC_OK) return st;
  if (!std::isfinite(cache_bias) && !(cache_bias < 0.f))
    return fail(RC_ERR_ARG, "cache_bias must be finite or -inf");
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(RC_ERR_ARG, "softmax_scale must be finite and >= 0");
  if (workspace_bytes > 0 && !workspace) return fail(RC_ERR_ARG, "workspace_bytes > 0 with a NULL workspace");
  rc::AttnCall c{q, n_q, q_pos0, q_block0, q_block ? 1 : q_block_len, cache_bias, softmax_scale, out, lse, workspace,
                 workspace_bytes};
  c.q_block_ids = q_block;
  c.same_block = mask == RC_MASK_SAME_BLOCK;
  c.precision = r->kv_dtype == RC_FP8_E4M3 ? attention_precision(r, g_precision.load(), q_block, n_q, q_block0,
                                                                   c.q_block_len, mask, cache_bias)
                                            : RC_PRECISION_AUTO;
  hipError_t e = rc::launch_chunk_attention(view(r), c, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "chunk attention");
  return ok();
}

rc_status rc_chunk_attention(const rc_ring* r, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                             int32_t q_block_len, float cache_bias, float softmax_scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return rc_chunk_attention_ex(r, q, n_q, q_pos0, nullptr, q_block0, q_block_len, RC_MASK_BLOCK_CAUSAL, cache_bias,
                               softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

size_t rc_key_mass_workspace_bytes(const rc_ring* r, int32_t n_q) {
  if (check_ring(r) != RC_OK || n_q < 1) return 0;
  return rc::key_mass_workspace_bytes(view(r), n_q);
}

namespace {
rc_status key_mass_impl(const rc_ring* r, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                        int32_t q_block_len, float cache_bias, float softmax_scale, const float* lse,
                        const int32_t* ranges, int32_t n_ranges, float* mass, void* workspace,
                        size_t workspace_bytes, void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if (!rc::key_mass_supported(r->kv_dtype, r->head_dim))
    return fail(RC_ERR_UNSUPPORTED, "key mass is built for FP8 rings only");
  if (!q || !lse || !mass) return fail(RC_ERR_ARG, "q / lse / mass is NULL");
  if (reinterpret_cast<uintptr_t>(q) & 15u) return fail(RC_ERR_ARG, "q must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(mass)) & 3u)
    return fail(RC_ERR_ARG, "lse and mass must be 4-byte aligned");
  if (n_q < 1) return fail(RC_ERR_ARG, "n_q must be >= 1 (got %d)", n_q);
  if (q_block_len < 1) return fail(RC_ERR_ARG, "q_block_len must be >= 1 (got %d)", q_block_len);
  if (static_cast<long long>(q_pos0) + n_q - 1 > INT32_MAX) return fail(RC_ERR_ARG, "positions overflow int32");
  if (static_cast<long long>(q_block0) + (n_q - 1) / q_block_len > INT32_MAX)
    return fail(RC_ERR_ARG, "query blocks overflow int32");
  if (!std::isfinite(cache_bias) && !(cache_bias < 0.f))
    return fail(RC_ERR_ARG, "cache_bias must be finite or -inf");
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(RC_ERR_ARG, "softmax_scale must be finite and >= 0");
  const size_t need = rc::key_mass_workspace_bytes(view(r), n_q);
  if (!workspace || workspace_bytes < need)
    return fail(RC_ERR_ARG, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(RC_ERR_ARG, "workspace must be 16-byte aligned");
  if (n_ranges < 0 || n_ranges > rc::kMassRanges)
    return fail(RC_ERR_ARG, "n_ranges must be in 0..%d (got %d)", rc::kMassRanges, n_ranges);
  if (n_ranges > 0 && !ranges) return fail(RC_ERR_ARG, "ranges is NULL");
  for (int i = 0; i < n_ranges; ++i)
    if (ranges[2 * i] < 0 || ranges[2 * i] >= ranges[2 * i + 1] || ranges[2 * i + 1] > r->n_slots)
      return fail(RC_ERR_ARG, "range %d [%d, %d) must satisfy 0 <= lo < hi <= n_slots (%d)", i, ranges[2 * i],
                  ranges[2 * i + 1], r->n_slots);
  rc::AttnCall c{q, n_q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale, nullptr, nullptr, workspace,
                 workspace_bytes};
  hipError_t e = rc::launch_key_mass(view(r), c, lse, mass, ranges, n_ranges, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "key mass");
  return ok();
}
}  // namespace

rc_status rc_key_mass(const rc_ring* r, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                      int32_t q_block_len, float cache_bias, float softmax_scale, const float* lse, float* mass,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return key_mass_impl(r, q, n_q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale, lse, nullptr, 0, mass,
                       workspace, workspace_bytes, stream);
}

rc_status rc_key_mass_slots(const rc_ring* r, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                            int32_t q_block_len, float cache_bias, float softmax_scale, const float* lse,
                            const int32_t* ranges, int32_t n_ranges, float* mass, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (n_ranges < 1) return fail(RC_ERR_ARG, "n_ranges must be >= 1 (got %d)", n_ranges);
  return key_mass_impl(r, q, n_q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale, lse, ranges, n_ranges,
                       mass, workspace, workspace_bytes, stream);
}

rc_status rc_ring_advance(rc_ring* r, int32_t n) {
  if (!r) return fail(RC_ERR_ARG, "ring is NULL");
  if (r->n_slots < 1 || r->n_anchor < 0 || r->n_memory < 0 ||
      static_cast<long long>(r->n_anchor) + r->n_memory >= r->n_slots)
    return fail(RC_ERR_ARG, "bad n_slots / n_anchor / n_memory (%d / %d / %d)", r->n_slots, r->n_anchor,
                r->n_memory);
  rc_status st = check_state(r);
  if (st != RC_OK) return st;
  if (r->n_cur == 0 || n != r->n_cur)
    return fail(RC_ERR_STATE, "advance(%d) needs n == n_cur > 0 (n_cur %d)", n, r->n_cur);
  r->head = step_slot(r, r->head, n);
  r->n_hist = std::min(r->n_hist + n, ring_end(r));
  r->n_cur = 0;
  return ok();
}

rc_status rc_debug_visibility(const rc_ring* r, int32_t n_q, int32_t q_block0, int32_t q_block_len, uint8_t* mask,
                              void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if (!mask) return fail(RC_ERR_ARG, "mask is NULL");
  if (n_q < 1 || q_block_len < 1) return fail(RC_ERR_ARG, "n_q and q_block_len must be >= 1");
  hipError_t e = rc::launch_debug_visibility(view(r), n_q, q_block0, q_block_len, mask, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "visibility");
  return ok();
}

size_t rc_debug_tile_classes_bytes(const rc_ring* r, int32_t n_q) {
  if (check_ring(r) != RC_OK || n_q < 1) return 0;
  return rc::debug_tile_classes_bytes(view(r), n_q);
}

rc_status rc_debug_tile_classes(const rc_ring* r, int32_t n_q, int32_t q_block0, int32_t q_block_len, int32_t mask,
                                float cache_bias, uint8_t* classes, size_t classes_bytes, void* stream) {
  rc_status st = check_ring(r);
  if (st != RC_OK) return st;
  if (!classes) return fail(RC_ERR_ARG, "classes is NULL");
  if (n_q < 1 || q_block_len < 1) return fail(RC_ERR_ARG, "n_q and q_block_len must be >= 1");
  if (mask != RC_MASK_BLOCK_CAUSAL && mask != RC_MASK_SAME_BLOCK) return fail(RC_ERR_ARG, "unknown mask %d", mask);
  if (!std::isfinite(cache_bias)) return fail(RC_ERR_ARG, "cache_bias must be finite");
  const size_t need = rc::debug_tile_classes_bytes(view(r), n_q);
  if (classes_bytes < need) return fail(RC_ERR_ARG, "classes holds %zu bytes, %zu needed", classes_bytes, need);
  hipError_t e = rc::launch_debug_tile_classes(view(r), n_q, q_block0, q_block_len, mask == RC_MASK_SAME_BLOCK,
                                               cache_bias, classes, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "tile classes");
  return ok();
}

const char* rc_last_error(void) { return g_err.c_str(); }

}  // extern "C"
