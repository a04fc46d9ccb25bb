// Block-causal chunk attention over an FP8 ring cache (gfx950, FP8 MFMA).
//
// Each call attends the chunk's new queries over every cached slot (Runway
// Characters, abstract), with a scalar bias added to the logits of earlier
// blocks (video-conductor, "Plastic Windows") and a block-causal mask
// (StreamLTX project page, Training).
//
// Work split.  A workgroup owns 128 queries of one head and runs 8 waves:
// 4 query waves of 32 x 2 key halves.  Half 1 walks the 128-slot tiles
// 0, 2, ..., half 0 the tiles 1, 3, ...; the two waves of a pair (same
// queries, different key halves) share the preparation of their queries and,
// at the end, the merge of their softmax states through LDS (each finishes
// half of the head dimension).  Tiles move global -> LDS with direct loads,
// double-buffered, one workgroup barrier per tile.
//
// Formulation.  S^T = K Q^T with 16x16x128 FP8 MFMAs: one instruction covers
// the whole head dimension of 16 slots x 16 queries, and every lane ends up
// holding 2 queries (one per 16-query block of its wave) and 4 slots per
// MFMA, so each per-slot factor read from LDS serves two queries (half the
// table reads of a one-query-per-lane layout).  K rows are fed to the MFMA in
// a permuted order so that lane group g = lane / 16 holds the 32 slots
// 32g .. 32g + 31 of the tile: the probabilities then sit exactly where the
// B operand of the P V MFMA (16x16x128, the reduction over the tile's 128
// slots) wants them, and V^T is read in natural slot order.
//
// Scales.  Queries are rotated (RoPE) and quantised with one power-of-two
// scale per (query, head), applied by the MFMA's E8M0 operand scale, so the
// accumulator is (k_code . q) with no per-query factor left over.  With the
// per-slot K and V scales, one logit in log2 units is
//   y = c s_k (Kc . q) + bias2,   c = softmax_scale log2(e),
// and V's scale is folded into the exponent (it varies along the reduction
// axis of P V):  P~ = 2^(y + log2 s_v - m) = p s_v,  l += P~ / s_v,  so
// O = sum P~ Vc needs no rescaling.  Per slot A = c s_k, C = log2(s_v) / A
// (the accumulator's start value) and 1/s_v are tabulated once per tile.
// The stabiliser m is raised only when a half-tile's maximum passes it by
// tau = 8 (log2), so P~ <= 256 stays inside e4m3 and O rescales are rare.
//
// Precision.  FP8 Q and P carry 3 mantissa bits each; the output error they
// cause shrinks like 1 / sqrt(effective number of keys).  Calls whose queries
// see few keys (the host bounds the effective key count from the ring state
// and the bias) run the two-term instantiation: Q and P are each split into
// two FP8 terms (codes of the value, then codes of the residual at 1/16 of the
// scale), which doubles both MFMA passes; it handles one 16-query block per
// pass over the tiles so that its extra operands stay in registers.
#include <cmath>
#include <type_traits>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void glb_void;

constexpr int kT = 128;        // slots per tile
constexpr int kHalves = 2;     // key halves per workgroup
constexpr int kQSub = 4;       // query waves per key half
constexpr int kWaves = kQSub * kHalves;
constexpr int kThreads = kWaves * kWave;
constexpr int kQW = 32;        // queries per wave (two blocks of 16)
constexpr int kQT = kQW * kQSub;  // queries per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.f;             // lazy-rescale threshold, log2 units
constexpr float kMinVScale = 0x1p-60f;  // floor for log2 / reciprocal of s_v
constexpr float kMinA = 0x1p-90f;       // floor of A, so that C stays finite
constexpr int kOne = 127;               // E8M0 code of 1.0
constexpr int kLoShift = 4;             // residual terms carry 1/16 of the scale

struct F8Args {
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* slot_block;
  int N, H, v_ld;
  const uint16_t* q;
  int n_q, q_pos0, q_block0, q_block_len;
  const int32_t* q_block_ids;  // [n_q] or null
  int same_block;
  float bias_log2;   // cache_bias * log2(e) (0 for the same-block mask)
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  float* lse;
  float* part_o;    // [splits][n_q][H][D] when split
  float* part_lse;  // [splits][H][n_q]
  int n_qt, n_splits, tiles_per_split, n_tiles;
  int remap, n_items;
  int use_rope;
  RopeTable rope;
};

// LDS geometry of one tile of one key half: K rows [128][D] in a K stage
// buffer, V^T rows [D][128 slots] in a V stage buffer.  K and V stages are
// separate arrays so that the compiler's wait analysis for direct-to-LDS
// loads (kept per LDS variable) never makes a read of one wait for loads
// into the other.
template <int D>
struct Tile {
  static constexpr int k_cpr = D / 16;  // 16-byte chunks per K row
  static constexpr int k_bytes = kT * D;
  static constexpr int v_bytes = D * kT;
  static constexpr int k_instr = k_bytes / 16 / (kQSub * kWave);  // direct loads per wave
  static constexpr int v_instr = v_bytes / 16 / (kQSub * kWave);
  static constexpr int dma_instr = k_instr + v_instr;
};

// Per-slot factors of one tile of one key half (128 entries each, indexed by
// the slot's place in the tile), then a summary of each half-tile
// {any slot occupied, min block, max block over occupied slots, 0}.  The
// half-tile ht holds the slots 32g + 16ht + 0..15, g = 0..3: the slots whose
// scores one wave computes between two stabiliser checks.
constexpr int kFacA = 0, kFacC = kT, kFacIv = 2 * kT, kFacKb = 3 * kT, kFacSum = 4 * kT;
constexpr int kFacWords = 4 * kT + 8;

template <int D>
struct Lds {
  static constexpr int kstage = kHalves * Tile<D>::k_bytes;
  static constexpr int vstage = kHalves * Tile<D>::v_bytes;
  static constexpr int fac = kHalves * kFacWords;  // words per stage
  static constexpr int total = 2 * kstage + 2 * vstage + 2 * fac * 4 + 512;
  static_assert(total <= 160 * 1024, "LDS budget");
};

// XOR swizzles of 16-byte chunks against LDS bank conflicts.  A 16-lane
// pass of a K read takes one chunk column of the rows 32a + 4sb + b
// (a, b = 0..3); of a V^T read one chunk column of 16 consecutive rows.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128) return (((r >> 5) & 3) << 1) | ((r >> 1) & 1);
  else return (r >> 5) & 3;
}
__device__ __forceinline__ int v_swz(int r) { return (r >> 1) & 7; }

// K row fed to MFMA row m (0..15) for slot block sb (0..7) of the tile, so
// that output row 4g + i of lane group g is slot 32g + 4sb + i.
__device__ __forceinline__ int k_perm(int sb, int m) { return 32 * (m >> 2) + 4 * sb + (m & 3); }

// Buffer resource over `bytes` bytes at `base` (raw: no stride, no format
// conversion; loads past the end return zeros).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// 16 bytes per lane from the buffer at lane offset off + uniform offset soff
// straight into LDS (the wave's 64 lanes fill 1024 consecutive bytes).  The
// buffer form takes a 32-bit lane offset and a scalar offset; the global
// form of the same load takes a 64-bit vector address per load, whose
// registers the tile loop cannot spare.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_wave_base), 16, static_cast<int>(off),
                                           static_cast<int>(soff), 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v4f mfma16(v8i a, v8i b, v4f c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kOne, 0, sb);
}

// Maximum (or sum) of a per-query value over the four lanes that hold the
// same query (lanes n, n + 16, n + 32, n + 48), for the two query blocks at
// once: x0 / x1 hold block 0 / block 1 on entry and the results on exit.
template <bool MAX>
__device__ __forceinline__ void across_groups(float& x0, float& x1) {
  auto op = [](float p, float q) { return MAX ? fmaxf(p, q) : p + q; };
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  float m = op(__uint_as_float(s[0]), __uint_as_float(s[1]));  // lanes < 32: block 0, else block 1
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = op(__uint_as_float(t[0]), __uint_as_float(t[1]));
  const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  x0 = __uint_as_float(u[0]);
  x1 = __uint_as_float(u[1]);
}

// Four floats to four e4m3 codes written over `old` (both halves replaced).
__device__ __forceinline__ int cvt_fp8x4_over(float a, float b, float c, float d, int old) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Four floats to four e4m3 codes.  Both halves of the word are written, so
// the word the first conversion starts from is a's own bits (no register has
// to be cleared first).
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  return cvt_fp8x4_over(a, b, c, d, __float_as_int(a));
}

// Residual codes of four values whose first-term codes are `hi`:
// code((x - decode(hi)) * 16).
__device__ __forceinline__ int residual_fp8x4(float a, float b, float c, float d, int hi, int old) {
  const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  return cvt_fp8x4_over((a - h01.x) * 16.f, (b - h01.y) * 16.f, (c - h23.x) * 16.f, (d - h23.y) * 16.f, old);
}

template <bool MAX>
__device__ __forceinline__ int wave_minmax_i32(int v) {
  auto op = [](int x, int y) { return MAX ? max(x, y) : min(x, y); };
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false));  // row_ror 8
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(static_cast<int>(r16[0]), static_cast<int>(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(static_cast<int>(r32[0]), static_cast<int>(r32[1]));
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = static_cast<int>(r16[0]) + static_cast<int>(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return static_cast<int>(r32[0]) + static_cast<int>(r32[1]);
}

// Summary of a half-tile from the block ids of its 64 slots, one per lane
// (-1 = empty): {any slot occupied, min block, max block over the occupied
// slots, 0}.
__device__ __forceinline__ v4i half_tile_summary(int kb) {
  const bool kval = kb != -1;
  const uint64_t vb = __ballot(kval);
  const int kmin = wave_minmax_i32<false>(kval ? kb : INT32_MAX);
  const int kmax = wave_minmax_i32<true>(kval ? kb : INT32_MIN);
  return v4i{vb != 0ull ? 1 : 0, kmin, kmax, 0};
}

// Class of a half-tile (summary any, kmin, kmax over its occupied slots) for
// a wave whose queries' blocks span qb_lo .. qb_hi.  vis: some slot may be
// visible to some query (exact under the block-causal mask, a superset under
// the same-block mask); fast: every occupied slot is visible to every query
// with one bias value (or the bias is 0), so the per-score mask is skipped
// (empty slots need no mask: their factor-table entry starts the QK
// accumulator at -inf, so their probability is exactly 0); hist: fast with
// the bias on every score.
struct HalfTileClass {
  bool vis, fast, hist;
};
__device__ __forceinline__ HalfTileClass half_tile_class(int any, int kmin, int kmax, int qb_lo, int qb_hi,
                                                         bool same_block, bool bias_zero) {
  const bool all_same = qb_lo == qb_hi && any && kmin == qb_lo && kmax == qb_lo;
  if (same_block) return {any && kmin <= qb_hi && kmax >= qb_lo, all_same, false};
  const bool all_vis = any && kmax <= qb_lo;
  const bool all_hist = any && kmax < qb_lo;
  const bool fast = all_vis && (all_hist || all_same || bias_zero);
  return {any && kmin <= qb_hi, fast, fast && all_hist};
}

// Softmax state and Q operands of the query blocks one pass handles: NB = 2
// (both 16-query blocks of the wave, one FP8 term) or 1 (one block, with the
// residual term of Q).
template <int NDB, int NB>
struct BlkState {
  static constexpr int nb = NB;
  v4f o[NDB][NB];
  float m_run[NB], msub[NB];  // stabiliser; msub = m_run, or 0 while it is -inf
  float l_part[NB][2];
  v8i qf[NB];
  v8i ql[NB];
  int qsc[NB], qsc_lo[NB], qb[NB];
  __device__ BlkState() {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db][b] = v4f{0.f, 0.f, 0.f, 0.f};
      m_run[b] = -INFINITY;
      msub[b] = 0.f;
      l_part[b][0] = l_part[b][1] = 0.f;
    }
  }
};

// GEN: per-query block ids and the same-block mask (rc_chunk_attention_ex).
// TWO: two FP8 terms for Q and P (one query block per pass over the tiles).
template <int D, bool GEN, bool TWO>
__global__ __launch_bounds__(kThreads) void attn_fp8_kernel(F8Args a) {
  using T = Tile<D>;
  constexpr int NDB = D / 16;       // d blocks of the output
  constexpr int NG = D / 32;        // lane groups that hold K / Q data (4, or 2 for d 64)
  __shared__ __attribute__((aligned(16))) uint8_t ks0[Lds<D>::kstage];
  __shared__ __attribute__((aligned(16))) uint8_t ks1[Lds<D>::kstage];
  __shared__ __attribute__((aligned(16))) uint8_t vs0[Lds<D>::vstage];
  __shared__ __attribute__((aligned(16))) uint8_t vs1[Lds<D>::vstage];
  __shared__ __attribute__((aligned(16))) float fac0[Lds<D>::fac];
  __shared__ __attribute__((aligned(16))) float fac1[Lds<D>::fac];
  __shared__ double rev_lds[64];  // RoPE frequencies in revolutions per position

  asm volatile("" ::"s"(a.n_qt), "s"(a.n_splits), "s"(a.tiles_per_split), "s"(a.n_tiles), "s"(a.remap),
               "s"(a.n_items), "s"(a.v_ld), "s"(a.H), "s"(a.n_q), "s"(a.k), "s"(a.v), "s"(a.q),
               "s"(a.slot_block), "s"(a.k_scale), "s"(a.v_scale));
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int kh = wave / kQSub;  // key half
  const int wq = wave % kQSub;  // query wave of the half
  const int n16 = lane & 15;    // query of each block / MFMA row
  const int g = lane >> 4;      // lane group

  // ---- work item
  int item = blockIdx.x;
  if (a.remap) item = (item % 8) * (a.n_items / 8) + item / 8;
  const int qt = item % a.n_qt;
  const int hs = item / a.n_qt;
  const int split = hs % a.n_splits;
  const int h = hs / a.n_splits;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.n_tiles, t_begin + a.tiles_per_split);
  const int n_local = (max(t_end - t_begin, 0) + 1) / 2;  // steps (tiles per half, rounded up)
  // key half 1 takes the even tiles, key half 0 the odd ones: with an even
  // tile count the last tile, partly empty and masked when the ring is full,
  // goes to the key half whose waves issue first, so the two halves end
  // their loops closer together
  auto tile_of = [&](int li, int half) { return t_begin + 2 * li + (1 - half); };
  auto has_tile = [&](int li, int half) { return li < n_local && tile_of(li, half) < t_end; };
  const int t_safe = min(t_begin, a.n_tiles - 1);

  // ---- direct-load plan: the lane's byte offsets inside a tile.  Load j of
  //      a wave covers 1024 bytes: K rows whose swizzle does not depend on j
  //      (K load j is K load 0 plus 1024 j), and V^T rows 8 (wq v_instr + j)
  //      + lane / 8, whose swizzle depends on j only through its parity (V
  //      load j is the offset of its parity plus 8 j rows)
  uint32_t k_off0, v_off_par[2];
  {
    const int p = wq * T::k_instr * kWave + lane;
    const int r = p / T::k_cpr, cp = p % T::k_cpr;
    k_off0 = static_cast<uint32_t>(r * D + ((cp ^ k_swz<D>(r)) << 4));
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int pv = (wq * T::v_instr + par) * kWave + lane;
      const int rv = pv / 8, cv = pv % 8;
      v_off_par[par] = static_cast<uint32_t>((rv - 8 * par) * a.v_ld + ((cv ^ v_swz(rv)) << 4));
    }
  }
  static_assert(T::k_instr * kWave * 16 % (D * 32) == 0, "K swizzle independent of the load index");
  // this head's K rows [v_ld][D] and V^T rows [D][v_ld] (byte offsets < 2^31)
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(a.k + static_cast<size_t>(h) * a.v_ld * D,
                                                  static_cast<uint32_t>(a.v_ld) * D);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(a.v + static_cast<size_t>(h) * D * a.v_ld,
                                                  static_cast<uint32_t>(a.v_ld) * D);
  // the j-th of this wave's T::dma_instr direct loads of tile li (K blocks
  // first) into the K / V stage buffers kst / vst
  auto issue_j = [&](uint8_t* kst, uint8_t* vst, int li, int j) __attribute__((always_inline)) {
    const int tile = has_tile(li, kh) ? tile_of(li, kh) : t_safe;
    if (j < T::k_instr) {
      dma16(k_rsrc, k_off0, static_cast<uint32_t>(tile * kT * D + 1024 * j),
            kst + kh * T::k_bytes + (wq * T::k_instr + j) * 1024);
    } else {
      const int jv = j - T::k_instr;
      dma16(v_rsrc, v_off_par[jv & 1], static_cast<uint32_t>(tile * kT + 8 * jv * a.v_ld),
            vst + kh * T::v_bytes + (wq * T::v_instr + jv) * 1024);
    }
  };
  auto issue_k = [&](uint8_t* kst, int li) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < T::k_instr; ++j) issue_j(kst, nullptr, li, j);
  };
  auto issue_v = [&](uint8_t* vst, int li) __attribute__((always_inline)) {
#pragma unroll
    for (int j = T::k_instr; j < T::dma_instr; ++j) issue_j(nullptr, vst, li, j);
  };

  // ---- per-slot metadata for the factor tables.  Table f (half f / 2,
  //      half-tile f % 2) of every step is built by the two waves with wq =
  //      f: the key-half-0 wave writes the per-slot factors, the key-half-1
  //      wave the half-tile summary, so that neither half carries the whole
  //      table work into the step barrier.  Lane L handles slot
  //      32 (L / 16) + 16 (f % 2) + L % 16 of the tile.
  const int fh = wq >> 1, fht = wq & 1;
  const int fslot = 32 * g + 16 * fht + n16;
  float m_ks = 0.f, m_vs = 0.f;
  int m_kb = -1;
  auto meta_load = [&](int li, float& ks, float& vs, int& kb) __attribute__((always_inline)) {
    const int tile = has_tile(li, fh) ? tile_of(li, fh) : t_safe;
    const size_t s = static_cast<size_t>(tile) * kT + fslot;
    ks = a.k_scale[static_cast<size_t>(h) * a.v_ld + s];
    vs = a.v_scale[static_cast<size_t>(h) * a.v_ld + s];
    kb = a.slot_block[s];
  };
  const float c_mul = a.scale_log2;
  auto fac_write = [&](float* ftab, float ks, float vs, int kb) __attribute__((always_inline)) {
    float* tbl = ftab + fh * kFacWords;
    if (kh == 0) {
      const float vsc = fmaxf(vs, kMinVScale);
      const float A = fmaxf(c_mul * ks, kMinA);
      tbl[kFacA + fslot] = A;
      // an empty slot starts its QK accumulator at -inf: every path then
      // gives it probability 0 without a per-score mask
      tbl[kFacC + fslot] = kb == -1 ? -INFINITY : __builtin_amdgcn_logf(vsc) * __builtin_amdgcn_rcpf(A);
      tbl[kFacIv + fslot] = __builtin_amdgcn_rcpf(vsc);
      reinterpret_cast<int32_t*>(tbl)[kFacKb + fslot] = kb;
      return;
    }
    const v4i sm = half_tile_summary(kb);
    if (lane == 0) *reinterpret_cast<v4i*>(tbl + kFacSum + 4 * fht) = sm;
  };

  // ---- queries of this lane: block b (0, 1) holds query wq * 32 + 16 b + n16
  const int q_base = qt * kQT;
  const int wave_q0 = q_base + wq * kQW;
  const bool wave_active = wave_q0 < a.n_q;
  int qi[2];
  bool q_ok[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    qi[b] = wave_q0 + 16 * b + n16;
    q_ok[b] = qi[b] < a.n_q;
  }
  int my_qb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int qq = q_ok[b] ? qi[b] : min(wave_q0, a.n_q - 1);
    my_qb[b] = (GEN && a.q_block_ids) ? a.q_block_ids[qq] : a.q_block0 + qq / a.q_block_len;
  }

  // ---- loads, in the order they are waited for: the RoPE frequencies, the
  //      metadata of the first two steps, Q, the first tiles
  const double rev_lane = wave == 0 && lane < D / 2 ? a.rope.rev[lane] : 0.0;
  float m2_ks = 0.f, m2_vs = 0.f;
  int m2_kb = -1;
  meta_load(0, m2_ks, m2_vs, m2_kb);  // every wave builds a part of the tables
  meta_load(1, m_ks, m_vs, m_kb);
  constexpr int kQLoads = 4;  // 16-byte loads per block: d = 32 g .. 32 g + 31 as bf16
  v4u qraw[2][kQLoads];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const size_t row = (static_cast<size_t>(q_ok[b] ? qi[b] : 0) * a.H + h) * D + 32 * (g % NG);
#pragma unroll
    for (int r = 0; r < kQLoads; ++r) qraw[b][r] = *reinterpret_cast<const v4u*>(a.q + row + 8 * r);
  }
  issue_k(ks0, 0);
  issue_v(vs0, 0);

  if (wave == 0) rev_lds[lane] = rev_lane;

  wait_lgkm0();
  bare_barrier();  // the RoPE table is visible

  // ---- Q: rotate, scale by a power of two per query, quantise into S's
  //      operands (the blocks S holds; with NB = 1 also the residual codes)
  auto prep_q = [&](auto& S, int b0) __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    if constexpr (NB == 2) {
      // the waves wq of the two key halves hold the same queries: the wave of
      // key half kh rotates and quantises block kh only and takes the other
      // block's operands from its partner through LDS (the second stage
      // buffers, free until the first step issues its loads)
      const int bq = kh;
      const long long qpos = static_cast<long long>(a.q_pos0) + (bq ? qi[1] : qi[0]);
      const bool live = (bq ? q_ok[1] : q_ok[0]) && g < NG;
      float xb[32];
#pragma unroll
      for (int e = 0; e < 32; e += 2) {
        const uint32_t w = bq ? qraw[1][e / 8][(e / 2) % 4] : qraw[0][e / 8][(e / 2) % 4];
        const float x0 = __uint_as_float(w << 16);
        const float x1 = __uint_as_float(w & 0xFFFF0000u);
        float c, sn;
        rope_cs_hw(rev_lds[(32 * (g % NG) + e) >> 1], qpos, &c, &sn);
        xb[e] = live ? x0 * c - x1 * sn : 0.f;
        xb[e + 1] = live ? x0 * sn + x1 * c : 0.f;
      }
      float am0 = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) am0 = fmaxf(am0, fabsf(xb[e]));
      float am1 = am0;
      across_groups<true>(am0, am1);
      const int bexp = static_cast<int>((__float_as_uint(am0) >> 23) & 0xFF);
      const int code = am0 > 0.f ? max(bexp - 7, 1) : kOne;
      const float inv = __uint_as_float(static_cast<uint32_t>(254 - code) << 23);
      v8i own;
#pragma unroll
      for (int w = 0; w < 8; ++w)
        own[w] = cvt_fp8x4_over(xb[4 * w] * inv, xb[4 * w + 1] * inv, xb[4 * w + 2] * inv, xb[4 * w + 3] * inv, 0);
      // exchange: 8 operand words per (wave wq, block, lane) in the second K
      // stage, the scale codes in the second V stage
      int32_t* xq = reinterpret_cast<int32_t*>(ks1);
      int32_t* xc = reinterpret_cast<int32_t*>(vs1);
      static_assert(kQSub * 2 * kWave * 32 <= Lds<D>::kstage && kQSub * 2 * kWave * 4 <= Lds<D>::vstage,
                    "Q exchange");
      const int own_slot = (wq * 2 + bq) * kWave + lane;
      const int oth_slot = (wq * 2 + 1 - bq) * kWave + lane;
      *reinterpret_cast<v8i*>(xq + 8 * own_slot) = own;
      xc[own_slot] = code;
      wait_lgkm0();
      bare_barrier();  // both blocks' operands are in LDS
      const v8i oth = *reinterpret_cast<const v8i*>(xq + 8 * oth_slot);
      const int oth_code = xc[oth_slot];
      S.qf[0] = bq == 0 ? own : oth;
      S.qf[1] = bq == 0 ? oth : own;
      S.qsc[0] = bq == 0 ? code : oth_code;
      S.qsc[1] = bq == 0 ? oth_code : code;
      S.qb[0] = my_qb[0];
      S.qb[1] = my_qb[1];
      return;
    }
    float x[NB][32];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int bq = b0 + b;
      const long long qpos = static_cast<long long>(a.q_pos0) + (bq ? qi[1] : qi[0]);
      const bool live = (bq ? q_ok[1] : q_ok[0]) && g < NG;
#pragma unroll
      for (int e = 0; e < 32; e += 2) {
        const uint32_t w = bq ? qraw[1][e / 8][(e / 2) % 4] : qraw[0][e / 8][(e / 2) % 4];
        const float x0 = __uint_as_float(w << 16);
        const float x1 = __uint_as_float(w & 0xFFFF0000u);
        // a ring without RoPE has every frequency 0: cos 1, sin 0 exactly
        float c, sn;
        rope_cs_hw(rev_lds[(32 * (g % NG) + e) >> 1], qpos, &c, &sn);
        x[b][e] = live ? x0 * c - x1 * sn : 0.f;
        x[b][e + 1] = live ? x0 * sn + x1 * c : 0.f;
      }
    }
    float am[2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(x[b][e]));
      am[b] = m;
    }
    if constexpr (NB == 1) am[1] = am[0];
    across_groups<true>(am[0], am[1]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // scale 2^e with e = floor(log2 max|q|) - 7: codes of magnitude < 256
      const int bexp = static_cast<int>((__float_as_uint(am[b]) >> 23) & 0xFF);
      const int code = am[b] > 0.f ? max(bexp - 7, 1) : kOne;
      const float inv = __uint_as_float(static_cast<uint32_t>(254 - code) << 23);
      S.qsc[b] = code;
      S.qsc_lo[b] = max(code - kLoShift, 1);
      const bool lo_ok = code > kLoShift;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float x0 = x[b][4 * w] * inv, x1 = x[b][4 * w + 1] * inv;
        const float x2 = x[b][4 * w + 2] * inv, x3 = x[b][4 * w + 3] * inv;
        const int hi = cvt_fp8x4_over(x0, x1, x2, x3, 0);
        S.qf[b][w] = hi;
        if constexpr (NB == 1) S.ql[b][w] = lo_ok ? residual_fp8x4(x0, x1, x2, x3, hi, 0) : 0;
      }
      S.qb[b] = (b0 + b) ? my_qb[1] : my_qb[0];
    }
  };

  // ---- LDS byte offsets of this lane's operand reads inside a tile buffer:
  //      K row k_perm(sb, n16) = k_perm(0, n16) + 4 sb, chunks 2g, 2g + 1;
  //      V^T row 16 db + n16, chunks 2g, 2g + 1.  Both swizzles are the same
  //      for every sb / db of a lane.
  int k_lane_lo, k_lane_hi, v_lane_lo, v_lane_hi;
  {
    const int row = k_perm(0, n16);
    const int sw = k_swz<D>(row);
    k_lane_lo = row * D + (((2 * g) ^ sw) << 4);
    k_lane_hi = row * D + (((2 * g + 1) ^ sw) << 4);
    const int swv = v_swz(n16);
    v_lane_lo = n16 * kT + (((2 * g) ^ swv) << 4);
    v_lane_hi = n16 * kT + (((2 * g + 1) ^ swv) << 4);
  }

  int qb_lo = INT32_MAX, qb_hi = INT32_MIN;
#pragma unroll
  for (int b = 0; b < 2; ++b)
    if (q_ok[b]) {
      qb_lo = min(qb_lo, my_qb[b]);
      qb_hi = max(qb_hi, my_qb[b]);
    }
  qb_lo = __builtin_amdgcn_readfirstlane(wave_minmax_i32<false>(qb_lo));
  qb_hi = __builtin_amdgcn_readfirstlane(wave_minmax_i32<true>(qb_hi));
  const bool same_block = GEN && a.same_block != 0;

  // Wave-uniform class of half-tile ht from its summary sm (read from the
  // tables at kFacSum + 4 ht).
  auto classify = [&](const v4i sm, bool& vis, bool& fast, bool& hist) __attribute__((always_inline)) {
    const int any = __builtin_amdgcn_readfirstlane(sm.x);
    const int kmin = __builtin_amdgcn_readfirstlane(sm.y);
    const int kmax = __builtin_amdgcn_readfirstlane(sm.z);
    const HalfTileClass c = half_tile_class(any, kmin, kmax, qb_lo, qb_hi, same_block, a.bias_log2 == 0.f);
    vis = c.vis;
    fast = c.fast;
    hist = c.hist;
  };

  const int n_steps = n_local;

  // ---- the pieces of one tile for the query blocks held in S (NB = 2: both,
  //      one FP8 term; NB = 1: one block, with the residual terms).  kb / vb
  //      are this key half's K rows and V^T rows of the tile, tbl its factor
  //      tables.
  //
  // O^T += V^T P^T over the tile's 128 slots (psc: the operand scale of pk)
  auto pv = [&](auto& S, const uint8_t* vb, const auto& pk, int psc) __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    const uint8_t* vl = vb + v_lane_lo;
    const uint8_t* vh = vb + v_lane_hi;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const v4i lo = *reinterpret_cast<const v4i*>(vl + 16 * db * kT);
      const v4i hi = *reinterpret_cast<const v4i*>(vh + 16 * db * kT);
      const v8i vop = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int b = 0; b < NB; ++b) S.o[db][b] = mfma16(vop, pk[b], S.o[db][b], psc);
    }
  };
  // S'^T = K Q^T + C for half-tile ht (slot blocks sb = 4ht .. 4ht + 3); dma(sb)
  // may issue one of the next tile's direct loads between matrix instructions
  auto qk_half = [&](auto& S, const uint8_t* kb, const float* tbl, int ht, auto& s, auto&& dma)
                     __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    constexpr bool two = NB == 1;
    const uint8_t* kl = kb + k_lane_lo;
    const uint8_t* kh8 = kb + k_lane_hi;
    const float* tg = tbl + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sb = 4 * ht + j;
      v8i kop = {0, 0, 0, 0, 0, 0, 0, 0};
      if (g < NG) {
        const v4i lo = *reinterpret_cast<const v4i*>(kl + 4 * sb * D);
        const v4i hi = *reinterpret_cast<const v4i*>(kh8 + 4 * sb * D);
        kop = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
      const v4f cin = *reinterpret_cast<const v4f*>(tg + kFacC + 4 * sb);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[j][b] = mfma16(kop, S.qf[b], cin, S.qsc[b]);
        if constexpr (two) s[j][b] = mfma16(kop, S.ql[b], s[j][b], S.qsc_lo[b]);
      }
      dma(sb);
    }
  };
  // z = A S' (+ bias) - msub, the masks, the stabiliser check, P~ = 2^z with
  // l += P~ / s_v, and P~ to FP8 into pk (bytes 4 sb + i of the P V operand).
  // `common` tiles (both half-tiles visible to every query of the wave with
  // one bias value each) take the bias per half-tile; the others are masked
  // per score from the slots' blocks.  If half-tile 1 raises the stabiliser,
  // half-tile 0's probabilities (already FP8, relative to the old stabiliser)
  // are multiplied into O (V^T of the tile in vb) before O is rescaled.  The
  // two-term path ends the tile here: both halves' first-term codes, then
  // their residual codes, multiplied into O.
  auto soft_half = [&](auto& S, const float* tbl, const uint8_t* vb, int ht, bool common, bool hist_ht, auto& s,
                       auto& pk, auto& p1) __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    constexpr bool two = NB == 1;
    const float* tg = tbl + 32 * g;
    const float zb = common && hist_ht ? a.bias_log2 : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f af = *reinterpret_cast<const v4f*>(tg + kFacA + 4 * (4 * ht + j));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float zadd = zb - S.msub[b];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[j][b][i] = fmaf(s[j][b][i], af[i], zadd);
      }
    }
    if (!common) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i kb4 = *reinterpret_cast<const v4i*>(tg + kFacKb + 4 * (4 * ht + j));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int qb = S.qb[b];
          const int lo_qb = same_block ? qb : 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kb = kb4[i];
            const int cls = !GEN ? visibility_class(kb, qb)
                                 : (kb < lo_qb || kb > qb) ? kVisNone : (kb < qb ? kVisBias : kVisPlain);
            const float z = cls == kVisBias ? s[j][b][i] + a.bias_log2 : s[j][b][i];
            s[j][b][i] = cls == kVisNone ? -INFINITY : z;
          }
        }
      }
    }
    float tmax[2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float t0 = fmaxf(fmaxf(s[0][b][0], s[0][b][1]), s[0][b][2]);
      float t1 = fmaxf(fmaxf(s[1][b][0], s[1][b][1]), s[1][b][2]);
      float t2 = fmaxf(fmaxf(s[2][b][0], s[2][b][1]), s[2][b][2]);
      float t3 = fmaxf(fmaxf(s[3][b][0], s[3][b][1]), s[3][b][2]);
      t0 = fmaxf(fmaxf(t0, s[0][b][3]), s[1][b][3]);
      t2 = fmaxf(fmaxf(t2, s[2][b][3]), s[3][b][3]);
      tmax[b] = fmaxf(fmaxf(t0, t1), fmaxf(t2, t3));
    }
    if constexpr (NB == 1) tmax[1] = tmax[0];

    // raise the stabiliser only when the half-tile maximum passes it by
    // tau, and only for the queries whose own maximum does: a query's
    // stabiliser and its rounding never depend on the other queries of its
    // wave (a raise in the second half-tile multiplies every query's
    // first-half probabilities into O early, which changes only the order
    // of one fp32 accumulation for the others).  A query's maximum passes
    // the threshold iff one of its four lanes' maxima does, so the lanes
    // test their own maxima first and the maxima are combined across the
    // lane groups only when some lane passes.
    bool lane_own = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) lane_own = lane_own || tmax[b] + S.msub[b] > S.m_run[b] + kTau;
    if (__ballot(lane_own) != 0ull) {
      across_groups<true>(tmax[0], tmax[1]);
      bool own[2] = {false, false};
#pragma unroll
      for (int b = 0; b < NB; ++b) own[b] = tmax[b] + S.msub[b] > S.m_run[b] + kTau;
      if (ht == 1) {  // the first half's P~ belong to the old stabiliser
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int w = 4; w < 8; ++w) pk[b][w] = 0;
        pv(S, vb, pk, kOne);
        if constexpr (two) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b)
              pk[b][j] = residual_fp8x4(p1[j][b][0], p1[j][b][1], p1[j][b][2], p1[j][b][3], pk[b][j], 0);
          pv(S, vb, pk, kOne - kLoShift);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pk[b][w] = 0;
            if constexpr (two) p1[w][b] = v4f{0.f, 0.f, 0.f, 0.f};  // no residual left either
          }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float m_new = own[b] ? fmaxf(S.m_run[b], tmax[b] + S.msub[b]) : S.m_run[b];
        const float alpha = !own[b] ? 1.f
                            : S.m_run[b] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S.m_run[b] - m_new);
        S.l_part[b][0] *= alpha;
        S.l_part[b][1] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) S.o[db][b] *= alpha;
        const float shift = !own[b] || m_new == -INFINITY ? 0.f : m_new - S.msub[b];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j][b] -= shift;
        S.m_run[b] = m_new;
        S.msub[b] = m_new == -INFINITY ? 0.f : m_new;
      }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sb = 4 * ht + j;
      const v4f iv = *reinterpret_cast<const v4f*>(tg + kFacIv + 4 * sb);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[j][b][i] = __builtin_amdgcn_exp2f(s[j][b][i]);
          S.l_part[b][i & 1] = fmaf(s[j][b][i], iv[i], S.l_part[b][i & 1]);
        }
        pk[b][sb] = cvt_fp8x4(s[j][b][0], s[j][b][1], s[j][b][2], s[j][b][3]);
        if constexpr (two) {
          if (ht == 0) p1[j][b] = s[j][b];
        }
      }
    }
    if constexpr (two) {
      if (ht == 1) {
        pv(S, vb, pk, kOne);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            pk[b][j] = residual_fp8x4(p1[j][b][0], p1[j][b][1], p1[j][b][2], p1[j][b][3], pk[b][j], 0);
            pk[b][4 + j] = residual_fp8x4(s[j][b][0], s[j][b][1], s[j][b][2], s[j][b][3], pk[b][4 + j], 0);
          }
        pv(S, vb, pk, kOne - kLoShift);
      }
    }
  };

  // ---- per step, one barrier, then each wave runs its tile's half-tiles and
  //      P V, issuing its share of the next tile's direct loads between its QK
  //      matrix instructions.
  auto step = [&](auto& S, uint8_t* kc, uint8_t* vc, uint8_t* kn, uint8_t* vn, float* fcur, float* fnxt, int st)
                  __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    wait_vm<0>();
    wait_lgkm0();
    bare_barrier();  // tile st and its tables are visible; every wave is done with kn / vn
    const bool more = st + 1 < n_steps;
    const float* tbl = fcur + kh * kFacWords;
    const uint8_t* kb = kc + kh * T::k_bytes;
    const uint8_t* vb = vc + kh * T::v_bytes;
    // the summaries are read before the next tile's table work, which then
    // covers their latency
    const v4i sm0 = *reinterpret_cast<const v4i*>(tbl + kFacSum);
    const v4i sm1 = *reinterpret_cast<const v4i*>(tbl + kFacSum + 4);
    if (more) {
      fac_write(fnxt, m_ks, m_vs, m_kb);
      if (st + 2 < n_steps) meta_load(st + 2, m_ks, m_vs, m_kb);
    }
    bool vis[2], fast[2], hist[2];
    classify(sm0, vis[0], fast[0], hist[0]);
    classify(sm1, vis[1], fast[1], hist[1]);
    if (!wave_active || !has_tile(st, kh) || (!vis[0] && !vis[1])) {
      if (more) {
        issue_k(kn, st + 1);
        issue_v(vn, st + 1);
      }
      return;
    }
    // past the last step the loads have no tile of their own: they reload a
    // valid one into the buffer nobody reads, so every wave issues the same
    // loads (the compiler then needs no waits of its own)
    auto dma = [&](int sb) __attribute__((always_inline)) {
      if (sb < T::dma_instr) issue_j(kn, vn, st + 1, sb);
    };
    const bool common = vis[0] && vis[1] && fast[0] && fast[1];
    v8i pk[NB];
    v4f p1[4][NB];  // fp32 probabilities of the first half (residual codes)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      v4f s[4][NB];
      qk_half(S, kb, tbl, ht, s, dma);
      soft_half(S, tbl, vb, ht, common, hist[ht], s, pk, p1);
    }
    if constexpr (NB == 2) pv(S, vb, pk, kOne);
  };

  // Merge the two key halves through LDS (the stage buffers are free then)
  // and store the outputs of the blocks in `S` (block b of S is query block
  // b0 + b of the wave).  Each key half finishes half of the d blocks: it
  // hands its stabilisers, sums and the other half's O to its partner and
  // takes the partner's for its own half, so both waves of a pair share the
  // merge and the stores.
  auto finish = [&](auto& S, int b0) __attribute__((always_inline)) {
    constexpr int NB = std::remove_reference_t<decltype(S)>::nb;
    constexpr int kHd = NDB / 2;           // d blocks per key half
    constexpr int kXh = 4 + 8 * kHd;       // words one key half hands over, per lane
    constexpr int kXw = 2 * kXh + 4;       // per lane (padded against bank conflicts)
    static_assert(kWave * kXw * 4 <= Lds<D>::kstage && kWave * kXw * 4 <= Lds<D>::vstage, "merge buffer");
    float l_sum[2];
#pragma unroll
    for (int b = 0; b < NB; ++b) l_sum[b] = S.l_part[b][0] + S.l_part[b][1];
    __syncthreads();
    uint8_t* xbuf = wq == 0 ? ks0 : wq == 1 ? ks1 : wq == 2 ? vs0 : vs1;
    float* xch = reinterpret_cast<float*>(xbuf) + lane * kXw;
    // key half kh finishes d blocks kh kHd .. kh kHd + kHd - 1 and hands over
    // the others.  The accumulators are chosen by value (a wave-uniform
    // select per register), never by a computed index, so they stay in
    // registers.
    const bool k0 = kh == 0;
    {
      float* w = xch + (k0 ? 0 : kXh);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        w[b] = S.m_run[b];
        w[2 + b] = l_sum[b];
#pragma unroll
        for (int i = 0; i < kHd; ++i)
          *reinterpret_cast<v4f*>(w + 4 + 8 * i + 4 * b) = k0 ? S.o[kHd + i][b] : S.o[i][b];
      }
    }
    __syncthreads();
    if (!wave_active) return;
    // every read first (one wait for all of them), then the arithmetic
    const float* r = xch + (k0 ? kXh : 0);
    const v4f ml = *reinterpret_cast<const v4f*>(r);
    v4f ox[kHd][NB];
#pragma unroll
    for (int i = 0; i < kHd; ++i)
#pragma unroll
      for (int b = 0; b < NB; ++b) ox[i][b] = *reinterpret_cast<const v4f*>(r + 4 + 8 * i + 4 * b);
    v4f mine[kHd][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float m1 = ml[b], l1 = ml[2 + b];
      const float mm = fmaxf(S.m_run[b], m1);
      const float a0 = S.m_run[b] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S.m_run[b] - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      // the same expression on both halves (key half 0's terms first), so the
      // two halves of a row are normalised by bit-identical sums
      const float ah0 = k0 ? a0 : a1, lh0 = k0 ? l_sum[b] : l1;
      const float ah1 = k0 ? a1 : a0, lh1 = k0 ? l1 : l_sum[b];
      l_sum[b] = ah0 * lh0 + ah1 * lh1;
#pragma unroll
      for (int i = 0; i < kHd; ++i) mine[i][b] = a0 * (k0 ? S.o[i][b] : S.o[kHd + i][b]) + a1 * ox[i][b];
      S.m_run[b] = mm;
    }
    // the lane holds d = 16 db + 4 g + 0..3 of its queries
    if constexpr (NB == 2) {
      across_groups<false>(l_sum[0], l_sum[1]);
    } else {
      float t1 = l_sum[0];
      across_groups<false>(l_sum[0], t1);
    }
    const int d0 = (k0 ? 0 : 16 * kHd) + 4 * g;  // first d of the lane's stores
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int qq = (b0 + b) ? qi[1] : qi[0];
      if (!((b0 + b) ? q_ok[1] : q_ok[0])) continue;
      const bool any = S.m_run[b] != -INFINITY && l_sum[b] > 0.f;
      const float osc = any ? 1.f / l_sum[b] : 0.f;
      const float lse_v = any ? (S.m_run[b] + __log2f(l_sum[b])) * kLn2 : -INFINITY;
      if (a.n_splits == 1) {
        uint16_t* orow = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(qq) * a.H + h) * D + d0;
#pragma unroll
        for (int i = 0; i < kHd; ++i) {
          const v4f r4 = mine[i][b] * osc;
          *reinterpret_cast<uint2*>(orow + 16 * i) = make_uint2(pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3]));
        }
        if (k0 && a.lse && g == 0) a.lse[static_cast<size_t>(h) * a.n_q + qq] = lse_v;
      } else {
        float* po = a.part_o + ((static_cast<size_t>(split) * a.n_q + qq) * a.H + h) * D + d0;
#pragma unroll
        for (int i = 0; i < kHd; ++i) *reinterpret_cast<v4f*>(po + 16 * i) = mine[i][b] * osc;
        if (k0 && g == 0) a.part_lse[(static_cast<size_t>(split) * a.H + h) * a.n_q + qq] = lse_v;
      }
    }
  };

  auto run = [&](auto& S) __attribute__((always_inline)) {
    for (int st = 0; st < n_steps; st += 2) {
      step(S, ks0, vs0, ks1, vs1, fac0, fac1, st);
      if (st + 1 < n_steps) step(S, ks1, vs1, ks0, vs0, fac1, fac0, st + 1);
    }
  };

  if constexpr (!TWO) {
    BlkState<NDB, 2> S;
    prep_q(S, 0);
    fac_write(fac0, m2_ks, m2_vs, m2_kb);
    run(S);
    finish(S, 0);
  } else {
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) {
        // restart the tile pipeline for the second query block (every wave
        // is past the merge, so the stage buffers are free)
        __syncthreads();
        meta_load(0, m2_ks, m2_vs, m2_kb);
        meta_load(1, m_ks, m_vs, m_kb);
        issue_k(ks0, 0);
        issue_v(vs0, 0);
      }
      BlkState<NDB, 1> S;
      prep_q(S, pass);
      fac_write(fac0, m2_ks, m2_vs, m2_kb);
      run(S);
      finish(S, pass);
    }
  }
}

// Merge split partials (each normalised by its own sum) in fixed split order.
template <int D>
__global__ __launch_bounds__(256) void combine_fp8_kernel(const float* part_o, const float* part_lse, int n_splits,
                                                          int n_q, int H, uint16_t* out, float* lse) {
  const int row = blockIdx.x * (256 / 32) + threadIdx.x / 32;
  const int lane = threadIdx.x % 32;
  if (row >= n_q * H) return;
  const int qi = row / H, h = row % H;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, part_lse[(static_cast<size_t>(s) * H + h) * n_q + qi]);
  float acc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float ls = part_lse[(static_cast<size_t>(s) * H + h) * n_q + qi];
      const float w = ls == -INFINITY ? 0.f : __expf(ls - mx);
      wsum += w;
      const float* po = part_o + ((static_cast<size_t>(s) * n_q + qi) * H + h) * D;
#pragma unroll
      for (int e = 0; e < D / 32; ++e) acc[e] += w * po[lane + 32 * e];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < D / 32; ++e) out[static_cast<size_t>(row) * D + lane + 32 * e] = f32_to_bf16(acc[e] * inv);
  if (lse && lane == 0) lse[static_cast<size_t>(h) * n_q + qi] = mx == -INFINITY ? -INFINITY : mx + logf(wsum);
}

// One wave per (query wave w, tile t, half-tile ht) of an FP8 attention call
// over the whole ring: the class the attention kernel gives that half-tile,
// from the same summary and rules (the wave's 32 queries 32 w .. 32 w + 31,
// their blocks q_block0 + q / q_block_len), as bits vis | fast << 1 | hist << 2.
__global__ __launch_bounds__(kWave) void tile_class_kernel(const int32_t* slot_block, int n_tiles, int n_q,
                                                           int q_block0, int q_block_len, int same_block,
                                                           int bias_zero, uint8_t* out) {
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const int ht = item & 1;
  const int t = (item >> 1) % n_tiles;
  const int w = (item >> 1) / n_tiles;
  const v4i sm = half_tile_summary(slot_block[t * kT + 32 * (lane >> 4) + 16 * ht + (lane & 15)]);
  int lo = INT32_MAX, hi = INT32_MIN;
  const int q = kQW * w + (lane & (kQW - 1));
  if (q < n_q) lo = hi = q_block0 + q / q_block_len;
  lo = wave_minmax_i32<false>(lo);
  hi = wave_minmax_i32<true>(hi);
  const HalfTileClass c = half_tile_class(sm.x, sm.y, sm.z, lo, hi, same_block != 0, bias_zero != 0);
  if (lane == 0) out[item] = static_cast<uint8_t>((c.vis ? 1 : 0) | (c.fast ? 2 : 0) | (c.hist ? 4 : 0));
}

template <int D>
hipError_t fp8_impl(const RingView& r, const AttnCall& c, int splits, hipStream_t s) {
  F8Args a{};
  a.k = static_cast<const uint8_t*>(r.k);
  a.v = static_cast<const uint8_t*>(r.v);
  a.k_scale = r.k_scale;
  a.v_scale = r.v_scale;
  a.slot_block = r.slot_block;
  a.N = r.N;
  a.H = r.H;
  a.v_ld = r.v_ld;
  a.q = static_cast<const uint16_t*>(c.q);
  a.n_q = c.n_q;
  a.q_pos0 = c.q_pos0;
  a.q_block0 = c.q_block0;
  a.q_block_len = c.q_block_len;
  a.q_block_ids = c.q_block_ids;
  a.same_block = c.same_block;
  const float sigma = c.softmax_scale != 0.f ? c.softmax_scale : 1.f / std::sqrt(static_cast<float>(r.d));
  a.scale_log2 = sigma * kLog2e;
  const float bias = c.same_block ? 0.f : c.cache_bias;
  a.bias_log2 = bias * kLog2e;
  a.out = c.out;
  a.lse = c.lse;
  a.n_qt = (c.n_q + kQT - 1) / kQT;
  a.n_tiles = (r.N + kT - 1) / kT;
  a.n_splits = splits;
  a.tiles_per_split = (a.n_tiles + splits - 1) / splits;
  a.use_rope = r.rope_base > 0.f;
  for (int j = 0; j < D / 2; ++j)
    a.rope.rev[j] = a.use_rope ? std::pow(static_cast<double>(r.rope_base), -2.0 * j / D) / (2.0 * M_PI) : 0.0;
  if (splits > 1) {
    a.part_o = static_cast<float*>(c.workspace);
    a.part_lse = a.part_o + static_cast<size_t>(splits) * c.n_q * r.H * D;
  }
  const int total = a.n_qt * r.H * splits;
  a.remap = (total % 8 == 0) ? 1 : 0;
  a.n_items = total;
  const bool gen = a.q_block_ids || a.same_block;
  const bool two = c.precision == 1;
  if (gen && two) hipLaunchKernelGGL((attn_fp8_kernel<D, true, true>), dim3(total), dim3(kThreads), 0, s, a);
  else if (gen) hipLaunchKernelGGL((attn_fp8_kernel<D, true, false>), dim3(total), dim3(kThreads), 0, s, a);
  else if (two) hipLaunchKernelGGL((attn_fp8_kernel<D, false, true>), dim3(total), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((attn_fp8_kernel<D, false, false>), dim3(total), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int rows = c.n_q * r.H;
  hipLaunchKernelGGL((combine_fp8_kernel<D>), dim3((rows + 7) / 8), dim3(256), 0, s, a.part_o, a.part_lse, splits,
                     c.n_q, r.H, static_cast<uint16_t*>(c.out), c.lse);
  return hipGetLastError();
}

}  // namespace

int fp8_attention_splits(const RingView& r, int n_q) {
  const int n_qt = (n_q + kQT - 1) / kQT;
  const int n_tiles = (r.N + kT - 1) / kT;
  const int items = n_qt * r.H;
  // Split the key range only when the grid is far below one workgroup per CU;
  // each split keeps at least 4 tiles (2 per key half).
  int splits = 1;
  while (items * splits * 2 <= 256 && (splits * 2) * 4 <= n_tiles) splits *= 2;
  return splits;
}

size_t debug_tile_classes_bytes(const RingView& r, int n_q) {
  return static_cast<size_t>((n_q + kQW - 1) / kQW) * ((r.N + kT - 1) / kT) * 2;
}

hipError_t launch_debug_tile_classes(const RingView& r, int n_q, int q_block0, int q_block_len, bool same_block,
                                     float cache_bias, uint8_t* out, hipStream_t s) {
  const int n_tiles = (r.N + kT - 1) / kT;
  const long long items = 2LL * n_tiles * ((n_q + kQW - 1) / kQW);
  if (items > INT32_MAX) return hipErrorInvalidValue;
  // the attention kernel's test: its bias in log2 units is exactly zero
  const float bias_log2 = (same_block ? 0.f : cache_bias) * kLog2e;
  hipLaunchKernelGGL(tile_class_kernel, dim3(static_cast<unsigned>(items)), dim3(kWave), 0, s, r.slot_block, n_tiles,
                     n_q, q_block0, q_block_len, same_block ? 1 : 0, bias_log2 == 0.f ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_fp8_attention(const RingView& r, const AttnCall& c, int splits, hipStream_t s) {
  return r.d == 128 ? fp8_impl<128>(r, c, splits, s) : fp8_impl<64>(r, c, splits, s);
}

}  // namespace rc
