/*
 * rc.h -- ring-cache chunk attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  It implements the attention hot path
 * of streaming autoregressive video diffusion as described in "Runway
 * Characters: Serving a 57B Video Diffusion Transformer for Real-Time
 * Conversation" (abstract): every chunk's new keys and values are written
 * once into a circular (ring) KV cache, with RoPE and FP8 quantisation applied
 * at write time, the cached keys are given a delta rotation when positions are
 * reset, and the chunk's queries attend over the whole cache on every call.
 * The attention adds a scalar cache bias to the logits of earlier blocks (the
 * "plastic window" of the video-conductor page, "Plastic Windows") and is
 * block-causal: full inside a block, backward-only across blocks (StreamLTX
 * project page, Training; "Why Live Video Generation Still Struggles With
 * Timing", transcript).
 *
 * Conventions shared by every call:
 *  - Device pointers point to GPU memory owned by the caller.  The library
 *    never allocates, frees or synchronises, and keeps no pointer after a call
 *    returns (the rc_ring struct holds the caller's pointers).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every device
 *    call is asynchronous on that stream.
 *  - Every argument and state check runs before anything is enqueued.  On a
 *    non-OK return nothing was enqueued and the host state in the rc_ring is
 *    unchanged; rc_last_error() describes the failure.  RC_ERR_HIP reports an
 *    error from the HIP runtime when enqueuing.
 *  - One ring is used from one host thread / stream at a time; there is no
 *    internal locking.  NaN or Inf inputs are outside the contract.
 */
#ifndef RC_H_
#define RC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RC_OK = 0,
  RC_ERR_ARG = 1,          /* invalid argument (null pointer, bad size, bad dtype) */
  RC_ERR_UNSUPPORTED = 2,  /* valid but not built (e.g. head_dim other than 64/128) */
  RC_ERR_STATE = 3,        /* call not allowed by the ring's host state */
  RC_ERR_HIP = 4           /* the HIP runtime reported an error */
} rc_status;

typedef enum {
  RC_F32 = 0,      /* float32 K and V                                  */
  RC_BF16 = 1,     /* bfloat16 K and V                                 */
  RC_FP8_E4M3 = 2  /* OCP e4m3fn codes (max 448) + float32 scales      */
} rc_dtype;

/*
 * One layer's ring cache.  The caller fills the geometry and the device
 * pointers, then calls rc_ring_init, which sets the host state.
 *
 * Device layout (sizes from rc_ring_sizes):
 *   k          [H][v_ld][d]     kv_dtype; row (h, s) is slot s of head h
 *   v          [H][d][v_ld]     kv_dtype, TRANSPOSED: v[h][j][s] is element
 *                               j of slot s; v_ld = rc_ring_v_ld(N) >= N
 *   k_scale    [H][v_ld] float  FP8 only: k = code * k_scale[h][s]
 *   v_scale    [H][v_ld] float  FP8 only: v = code * v_scale[h][s]
 *   slot_pos   [v_ld]   int32   token position of each slot
 *   slot_block [v_ld]   int32   block id of each slot, -1 = never written
 * Entries s in [N, v_ld) are padding: the kernels read them as empty slots
 * (block -1, scale 0, V 0) and never write them.
 * Anchor + sliding window (Why Live Video Generation Still Struggles With
 * Timing, transcript: the first chunk kept as a permanent anchor beside recent
 * history; StreamLTX project page, "Why a long take does not slow down": an
 * anchor next to a FIFO).  With n_anchor = A > 0 the first A tokens written
 * fill slots 0..A-1 and are never evicted; every later token goes to the
 * sliding part, slots A..N-1, used as a ring of N - A slots.  Writes then wrap
 * from slot N-1 to slot A instead of slot 0.  An anchored ring starts at slot 0
 * and its chunks hold at most N - A tokens.  Attention and re-rotation treat
 * anchor slots like any other written slot.
 * Content memory (StreamLTX project page, "Why a long take does not slow
 * down": an anchor, a content memory and a FIFO of recent blocks, each layer
 * scoring its own keys and keeping a top-M budget).  With n_memory = M > 0 the
 * last M slots, E = N - M .. N-1, are the memory and the sliding part is
 * A..E-1: writes wrap from E to A and a chunk holds at most E - A tokens.
 * rc_cache_write lets the history tokens it overwrites go; rc_cache_write_scored
 * first keeps the best of them in the memory.  Memory slots are read by
 * attention and moved by re-rotation like any other written slot.
 * Host state (maintained by the library; read it, do not write it):
 *   head       next slot to write
 *   n_hist     committed history tokens in the anchor and sliding part (<= E)
 *   n_cur      tokens of the current, not yet committed, chunk (0 = none)
 *   cur_pos0, cur_block   position of the current chunk's first token, its block
 *   n_mem      occupied memory slots; they are always slots E .. E + n_mem - 1
 *   max_block  largest block id written since rc_ring_init (-1: none); the FP8
 *              attention's automatic operand precision reads it
 *   pos_lo, pos_hi   least and greatest token position written since
 *              rc_ring_init, both moved by every re-rotation (pos_lo > pos_hi:
 *              nothing written); a bound of every cached slot's position,
 *              which rc_cache_rerotate keeps inside int32
 */
typedef struct rc_ring {
  int32_t n_slots;     /* N >= 1 */
  int32_t n_heads;     /* H >= 1 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t kv_dtype;    /* rc_dtype */
  float rope_base;     /* RoPE base (10000 on the pages' workloads); 0 = no RoPE */
  int32_t v_ld;        /* must equal rc_ring_v_ld(n_slots) */
  int32_t n_anchor;    /* A pinned slots at the start (0 = none); see below */
  int32_t n_memory;    /* M content-memory slots at the end (0 = none); A + M < N */
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  int32_t* slot_pos;
  int32_t* slot_block;
  int32_t head, n_hist, n_cur, cur_pos0, cur_block, n_mem, max_block, pos_lo, pos_hi;
} rc_ring;

/* Leading dimension of the transposed V buffer: N rounded up to 128 (a whole
   number of the attention's 128-slot tiles). */
int32_t rc_ring_v_ld(int32_t n_slots);

/*
 * Byte sizes of the six device buffers of a ring, written to out[0..5] in the
 * order k, v, k_scale, v_scale, slot_pos, slot_block (scales are 0 unless
 * FP8).  Returns RC_ERR_ARG / RC_ERR_UNSUPPORTED for a bad geometry.
 */
rc_status rc_ring_sizes(int32_t n_slots, int32_t n_heads, int32_t head_dim, int32_t kv_dtype,
                        size_t out[6]);

/*
 * Start an empty ring cache (Runway Characters, abstract: the KV cache is a
 * ring that every chunk writes once; an empty ring has no visible slot).
 * Validate the geometry and pointers, zero K, V and the scales, set every
 * slot_block to -1 and slot_pos to 0 (asynchronously on `stream`), and set the
 * host state: head = first_slot (0 <= first_slot < N - n_memory; 0 when
 * n_anchor > 0), n_hist = n_cur = n_mem = 0, max_block = -1, pos_lo =
 * INT32_MAX, pos_hi = INT32_MIN.  RC_ERR_ARG for
 * a null ring or pointer, a bad geometry or first_slot out of range.
 */
rc_status rc_ring_init(rc_ring* ring, int32_t first_slot, void* stream);

/*
 * Write n_new tokens into slots head + i, i < n_new, wrapping from E = N -
 * n_memory to n_anchor (so (head + i) mod N for the plain ring) (Runway
 * Characters, abstract: ring cache, RoPE and FP8 quantisation once per write).
 *   k_new, v_new  device [n_new][H][d], bfloat16 (float32 for an RC_F32 ring),
 *                 token-major as a QKV projection produces them
 *   pos0          position of token 0; token i has position pos0 + i
 *   block_id      block id (>= 0) recorded for every written slot
 * K is rotated by RoPE at its position; for FP8 rings each (head, token)
 * vector of K and of V is quantised with scale = max|x| / 448 (float32) and
 * codes = round-to-nearest-even(x / scale); for BF16 rings the values are
 * rounded to bfloat16.  slot_pos and slot_block are set for the written slots.
 * History slots overwritten by the write are evicted: n_hist becomes
 * min(n_hist, E - n_new).  Every denoising pass of one chunk writes again
 * before rc_ring_advance: while n_cur > 0, n_new, pos0 and block_id must repeat
 * the current chunk's, else RC_ERR_STATE.  Requires 1 <= n_new <= E - n_anchor.
 */
rc_status rc_cache_write(rc_ring* ring, const void* k_new, const void* v_new, int32_t n_new,
                         int32_t pos0, int32_t block_id, void* stream);

/*
 * Position reset (Runway Characters, abstract: a delta rotation when
 * positions reset).  Every slot with slot_block != -1 (history and the current
 * chunk) has its key rotated by delta: FP8 codes are dequantised, rotated,
 * and quantised again with a fresh absmax scale.  slot_pos += delta for those
 * slots, and cur_pos0 += delta when a chunk is current.  V is untouched.
 * Requires rope_base > 0.  RC_ERR_ARG when delta would take a cached
 * position (any position in pos_lo .. pos_hi) outside int32.
 */
rc_status rc_cache_rerotate(rc_ring* ring, int32_t delta, void* stream);

/*
 * Block-causal chunk attention of n_q queries over every cached slot: the
 * chunk's queries attend over the whole ring on every call (Runway
 * Characters, abstract), earlier blocks' logits take the scalar cache bias
 * (video-conductor, "Plastic Windows"), and the mask is full inside a block
 * and backward-only across blocks (StreamLTX project page, Training).
 *   q            device [n_q][H][d], bfloat16 (float32 for an RC_F32 ring),
 *                not yet rotated; query i has position q_pos0 + i and block
 *                q_block0 + i / q_block_len
 *   cache_bias   added to the scaled logit of every visible slot whose block
 *                is earlier than the query's (the plastic-window bias)
 *   softmax_scale  logit scale; 0 means 1/sqrt(d)
 *   out          device [n_q][H][d], same dtype as q
 *   lse          device [H][n_q] float32 natural-log sum of exp of the logits,
 *                or NULL
 *   workspace    device scratch of workspace_bytes (may be NULL / 0); more
 *                workspace lets the call split the key range over more
 *                workgroups when n_q is small
 * Slot s is visible to query i iff slot_block[s] != -1 and
 * slot_block[s] <= block(i).  logit = scale * (RoPE(q_i) . k_s) +
 * cache_bias * [slot_block[s] < block(i)].  A query that sees no slot gets
 * out = 0 and lse = -inf.  Requires n_q >= 1 and q_block_len >= 1.
 * RC_ERR_UNSUPPORTED for an RC_F32 ring with head_dim 128 (float32 rings are
 * a checking format; their attention kernel is built for head_dim 64 only).
 */
rc_status rc_chunk_attention(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0,
                             int32_t q_block0, int32_t q_block_len, float cache_bias,
                             float softmax_scale, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Masks of rc_chunk_attention_ex. */
typedef enum {
  RC_MASK_BLOCK_CAUSAL = 0, /* slot_block != -1 and slot_block <= block(i); bias on earlier blocks */
  RC_MASK_SAME_BLOCK = 1    /* slot_block == block(i) (>= 0); no bias */
} rc_mask;

/*
 * rc_chunk_attention with explicit query blocks and a choice of mask, for
 * the joint audio-video block (StreamLTX project page, Training and Data):
 *   q_block   device [n_q] int32 block id of every query (>= 0), or NULL for
 *             q_block0 + i / q_block_len.  Blocks of unequal length occur when
 *             the first block of a take carries one latent frame more (4 + 3k
 *             video and 26 + 25k audio frames).
 *   mask      RC_MASK_BLOCK_CAUSAL as rc_chunk_attention, or RC_MASK_SAME_BLOCK
 *             for the text cross-attention paths, where each block sees only
 *             the prompt of its own segment: text slots carry their segment's
 *             id as block id, queries their block's segment id, and slot s is
 *             visible to query i iff slot_block[s] == block(i); cache_bias is
 *             not applied.
 * Everything else as rc_chunk_attention (which is this call with q_block =
 * NULL and RC_MASK_BLOCK_CAUSAL).
 */
rc_status rc_chunk_attention_ex(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0,
                                const int32_t* q_block, int32_t q_block0, int32_t q_block_len, int32_t mask,
                                float cache_bias, float softmax_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Operand precision of the attention on FP8 rings, for the whole process (a
 * checking and measurement control; the default needs no call).  The FP8
 * attention quantises the rotated queries with one power-of-two scale per
 * (query, head) and the probabilities per score; each FP8 term keeps 3
 * mantissa bits, and the output error they cause falls like one over the
 * square root of the effective number of keys a query sees (Runway
 * Characters, abstract: FP8 KV cache; the rest of the attention's arithmetic
 * is the block-causal softmax of rc_chunk_attention).
 *   RC_PRECISION_AUTO      (0, default) one FP8 term for Q and for P when the
 *                          call's queries all lie in one block b >= max_block
 *                          (so every occupied slot is visible), the mask is
 *                          block-causal, and a lower bound of the effective
 *                          number of keys (n_b + n_<b w)^2 / (n_b + n_<b w^2)
 *                          reaches 2048, where w = exp(cache_bias), the
 *                          n_hist + n_cur + n_mem occupied slots split into
 *                          n_b slots of block b (at least n_cur when b is the
 *                          current chunk's block) and n_<b earlier ones, and
 *                          the bound is the minimum over the splits the ring
 *                          state allows; two terms (the codes of the residual
 *                          at 1/16 of the scale added) otherwise
 *   RC_PRECISION_TWO_TERM  (1) two terms for every call
 *   RC_PRECISION_ONE_TERM  (2) one term for every call
 * RC_ERR_ARG for any other mode.  Calls already enqueued are not affected.
 */
typedef enum { RC_PRECISION_AUTO = 0, RC_PRECISION_TWO_TERM = 1, RC_PRECISION_ONE_TERM = 2 } rc_precision;
rc_status rc_set_attention_precision(int32_t mode);

/* Workspace that lets rc_chunk_attention use its full key split for n_q queries. */
size_t rc_attention_workspace_bytes(const rc_ring* ring, int32_t n_q);

/*
 * rc_chunk_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call and the same result, with the key-split partials
 * kept in a fixed device array of the library (rc_attention_noalloc_limit()
 * bytes, 16 MiB, held by every GPU the library runs on until the process
 * ends) instead of a workspace argument.  The call allocates nothing; its
 * first call on a device looks up that device's array (the device current at
 * the call).  RC_ERR_ARG when the call would need more than the limit
 * (rc_attention_workspace_bytes(ring, n_q) bytes), otherwise the checks and
 * errors of rc_chunk_attention.  Calls that overlap on one GPU share the
 * array and race: serialise them (one stream per GPU).
 */
rc_status rc_chunk_attention_noalloc(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0,
                                     int32_t q_block0, int32_t q_block_len, float cache_bias, float softmax_scale,
                                     void* out, float* lse, void* stream);
size_t rc_attention_noalloc_limit(void);

/*
 * Commit the current chunk as history once its last denoising pass is done
 * (Runway Characters, abstract: each chunk's keys and values are written
 * once and then serve every later chunk from the ring).  Host only, nothing
 * is enqueued: head moves n slots on (wrapping from E to n_anchor), n_hist =
 * min(n_hist + n, E), n_cur = 0.  Requires n == n_cur > 0 (RC_ERR_STATE
 * otherwise, RC_ERR_ARG for a null ring).
 */
rc_status rc_ring_advance(rc_ring* ring, int32_t n);

/*
 * Attention mass per head and slot, the attention quality by which a layer
 * scores its keys (StreamLTX project page, "Why a long take does not slow
 * down"): mass[h][s] += sum over queries i of p_h(i, s), where p is the
 * block-causal softmax of rc_chunk_attention with the same arguments,
 * normalised by the lse that call returned.
 *   q, n_q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale
 *              as for rc_chunk_attention
 *   lse        device [H][n_q] float32: that call's lse output
 *   mass       device [H][v_ld] float32, accumulated into (the caller clears
 *              it); invisible slots and padding entries get += 0
 *   workspace  device scratch of rc_key_mass_workspace_bytes(ring, n_q) bytes
 * Products are taken in FP8 (queries quantised per 32 queries) like the
 * attention; every mass entry is summed by one wave in a fixed order (no
 * atomics), so results are reproducible.  FP8 rings only (RC_ERR_UNSUPPORTED
 * otherwise).
 */
rc_status rc_key_mass(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                      int32_t q_block_len, float cache_bias, float softmax_scale, const float* lse, float* mass,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * rc_key_mass for the slots of n_ranges (1..4) slot ranges only: the scored
 * write reads the scores of its candidates alone (the memory slots and the
 * slots the next write overwrites), so only those need the mass.
 *   ranges     host int32 pairs lo, hi with 0 <= lo < hi <= n_slots; the
 *              slots lo .. hi-1 of each range get their mass added exactly as
 *              rc_key_mass would add it (the same sums, bit for bit); every
 *              other entry of mass is left untouched
 * Arguments otherwise, workspace and errors as rc_key_mass; a bad range or
 * count is RC_ERR_ARG.
 */
rc_status rc_key_mass_slots(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0, int32_t q_block0,
                            int32_t q_block_len, float cache_bias, float softmax_scale, const float* lse,
                            const int32_t* ranges, int32_t n_ranges, float* mass, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace rc_key_mass needs for n_q queries (0 for a bad ring or n_q). */
size_t rc_key_mass_workspace_bytes(const rc_ring* ring, int32_t n_q);

/*
 * rc_cache_write with a scored content memory.  On the first pass of a chunk
 * (n_cur == 0) of a ring with n_memory = M > 0, the history tokens the write
 * will overwrite compete with the tokens in the memory for its M slots before
 * they are overwritten (StreamLTX project page, "Why a long take does not
 * slow down": each layer scores its keys on attention quality and temporal
 * diversity and keeps a top-M budget):
 *   key_score  device [H][v_ld] float32, finite and >= 0 (rc_key_mass of the
 *              previous chunk's queries, say).  A slot's score Q is the
 *              float64 sum of its H entries in head order.
 *   diversity  gamma in (0, 1].  The memory keeps the min(M, candidates)
 *              tokens that maximise the sum over blocks of
 *              sum_k Q_(k) gamma^k, Q_(0) >= Q_(1) >= ... the kept scores of
 *              one block: gamma = 1 is top-M by score, a smaller gamma
 *              spreads the memory over more blocks.  The choice is the greedy
 *              one: each block offers its best remaining token (higher Q,
 *              then lower slot) with gain Q gamma^c (c tokens of the block
 *              already kept; gamma^c the float32 product of c factors of the
 *              float32 gamma, left to right; the gain is the float64
 *              product); the largest gain is kept, ties to the smaller c, then
 *              the lower slot.
 *   workspace  device scratch of rc_cache_write_scored_workspace_bytes(ring,
 *              n_new) bytes
 * Kept tokens from the sliding part move (K, V, scales, position, block) into
 * the memory slots that hold no kept token, both taken in ascending slot
 * order; then the write proceeds as rc_cache_write.  n_mem becomes
 * min(M, n_mem + evicted history tokens).  Requires M + n_new <= 4096
 * (RC_ERR_UNSUPPORTED otherwise).  Without a memory, or on a later pass, this
 * is rc_cache_write (key_score and workspace are not read).
 */
rc_status rc_cache_write_scored(rc_ring* ring, const void* k_new, const void* v_new, int32_t n_new, int32_t pos0,
                                int32_t block_id, const float* key_score, float diversity, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace rc_cache_write_scored needs for a write of n_new tokens. */
size_t rc_cache_write_scored_workspace_bytes(const rc_ring* ring, int32_t n_new);

/*
 * The QKV projection with the cache write fused into its epilogue (Runway
 * Characters, abstract: FP8 GEMMs; RoPE and FP8 quantisation once per write).
 * For the n tokens of x:
 *   [q | k | v] = x W^T with FP8 operands: x is quantised per token with the
 *   cache's rule (scale = max|x_t| / 448, float32; codes round to nearest
 *   even), W is given as e4m3 codes with one float32 scale per row, and the
 *   products accumulate in float32.
 *   x        device [n][C] bfloat16 (the layer input); C a multiple of 128
 *   w        device [3 H d][C] e4m3 codes: rows 0 .. H d - 1 give q (head-
 *            major), then k, then v
 *   w_scale  device [3 H d] float32
 *   q_out    device [n][H][d] bfloat16: q, not rotated (rc_chunk_attention's
 *            q input)
 *   workspace  device scratch of rc_qkv_workspace_bytes(n, C) bytes
 * x, w, q_out and workspace must be 16-byte aligned, w_scale 4-byte aligned
 * (RC_ERR_ARG otherwise).
 * k and v are stored into the ring as rc_cache_write would store them (k
 * rotated at position pos0 + i, both quantised per (token, head), slot
 * metadata), from their float32 values: they never exist in HBM in another
 * form.  Same slots, state rules and errors as rc_cache_write.  FP8 rings with
 * head_dim 128 only (RC_ERR_UNSUPPORTED otherwise).
 */
rc_status rc_qkv_project_write(rc_ring* ring, const void* x, int32_t n, int32_t C, const uint8_t* w,
                               const float* w_scale, int32_t pos0, int32_t block_id, void* q_out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace rc_qkv_project_write needs for n tokens of width C. */
size_t rc_qkv_workspace_bytes(int32_t n, int32_t C);

/*
 * The visibility predicate used inside rc_chunk_attention, exported for
 * checking: mask[i][s] (device uint8 [n_q][N]) = 0 if slot s is invisible to
 * query i, 1 if visible without the bias (same block), 2 if visible with the
 * bias (earlier block).
 */
rc_status rc_debug_visibility(const rc_ring* ring, int32_t n_q, int32_t q_block0,
                              int32_t q_block_len, uint8_t* mask, void* stream);

/*
 * The FP8 attention kernel's own tile classes, exported for checking (the
 * decision that lets it skip the per-score mask; the masks themselves are
 * rc_chunk_attention's and rc_chunk_attention_ex's, defined there).  For a
 * call with n_q queries in blocks q_block0 + i / q_block_len, under mask
 * (RC_MASK_BLOCK_CAUSAL or RC_MASK_SAME_BLOCK) and cache_bias, over the whole
 * ring: classes (device uint8 [ceil(n_q / 32)][ceil(N / 128)][2]) holds for
 * each 32-query wave w, 128-slot tile t and half-tile h (the 64 slots
 * 128 t + 32 g + 16 h + 0..15, g = 0..3) the bits
 *   1  vis:  some slot may be visible to some query of the wave (exact under
 *            the block-causal mask; a superset under the same-block mask);
 *   2  fast: the half-tile has an occupied slot, and every occupied slot is
 *            visible to every query of the wave with one bias value (or
 *            cache_bias is 0): the per-score mask is skipped (empty slots get
 *            probability 0 without it);
 *   4  hist: fast, with the bias on every score.
 * classes_bytes >= rc_debug_tile_classes_bytes(ring, n_q), else RC_ERR_ARG;
 * RC_ERR_ARG also for a bad mask, a non-finite bias, n_q or q_block_len < 1.
 */
size_t rc_debug_tile_classes_bytes(const rc_ring* ring, int32_t n_q);
rc_status rc_debug_tile_classes(const rc_ring* ring, int32_t n_q, int32_t q_block0, int32_t q_block_len,
                                int32_t mask, float cache_bias, uint8_t* classes, size_t classes_bytes,
                                void* stream);

/* Thread-local description of the last error (empty string if none). */
const char* rc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RC_H_ */
