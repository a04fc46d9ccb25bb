// Block-causal chunk attention over the ring cache (gfx950, MFMA).
//
// Each call attends the chunk's new queries over every cached slot
// (Runway Characters, abstract), with a scalar bias added to the logits of
// earlier blocks (video-conductor, "Plastic Windows") and a block-causal mask
// (StreamLTX project page, Training).
//
// Work split.  A workgroup owns 128 queries of one head and runs 8 waves: 4
// query sub-tiles of 32 x 2 key halves.  Half k walks the tiles k, k+2, ...
// of 64 slots; at the end the two halves of each query sub-tile merge their
// softmax states through LDS.  Tiles reach LDS by direct global->LDS loads
// (no registers) three stages ahead; each half has its own stage buffers.
//
// Formulation.  A wave computes S^T = K Q^T with 32x32 MFMAs, so the
// accumulator gives every lane ONE query (column l % 32) and 32 slots: the
// online-softmax state (running max, running sum, output row) is per lane and
// the only cross-lane step is one swap with lane l ^ 32 (the other 32 slots
// of the same query).  The output stays transposed: O^T = V^T P^T.  The A
// operand of the first MFMA reads K rows in a permuted order chosen so that
// lane group g = l / 32 ends up holding slots 32g .. 32g+31 of the tile: the
// probabilities then sit in exactly the register order the P^T operand of the
// second MFMA needs, and V^T is read in natural slot order.
//
// Scales (FP8 cache).  With per-slot K and V scales and a per-workgroup Q
// scale, one logit in log2 units is  y0 = c * s_k[slot] * (Qc . Kc) + bias2
// with c = softmax_scale * log2(e) * s_q.  V's per-slot scale varies along the
// reduction axis of P V, so it is folded into the exponent:
//   y  = y0 + log2(s_v[slot]),   P~ = 2^(y - m) = p * s_v,   l += P~ / s_v
// so O = sum P~ Vc needs no further scaling and P~ <= 2^tau for the running
// stabiliser m.  Per slot, c*s_k, log2 s_v (+ bias2) and 1/s_v are computed
// once per tile into LDS; a score then costs one FMA, half a max, a subtract,
// an exp2, one FMA for the sum and half an FP8 conversion.  The stabiliser is
// only raised when a tile's maximum exceeds it by more than tau = 8 (log2),
// which keeps P~ <= 256 inside e4m3's range and makes O rescales rare.
//
// Masks.  A tile whose 64 slots are all visible to all of the wave's queries
// with one bias value takes the fast path; other tiles evaluate visibility
// and bias per (slot, query) from the slot's block id; tiles no query of the
// wave can see are skipped.  Slots are walked in physical order: softmax does
// not depend on slot order, so a wrapped ring needs no special case.
#include <cmath>
#include <type_traits>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
// LDS reads use native vector types: a 16-byte read then reaches the backend
// as one load that keeps its alias information, which the wait insertion
// needs to see that it does not depend on loads in flight to other stages.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void glb_void;

constexpr int kKT = 64;       // slots per tile
constexpr int kQW = 32;       // queries per wave
constexpr int kQSub = 4;      // query sub-tiles per workgroup
constexpr int kHalves = 2;    // key halves per workgroup
constexpr int kWaves = kQSub * kHalves;
constexpr int kThreads = kWaves * kWave;
constexpr int kQT = kQW * kQSub;  // queries per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.f;            // lazy-rescale threshold, log2 units
constexpr float kMinVScale = 0x1p-60f; // floor for log2 / reciprocal of s_v

template <int KV>
struct KvT {
  static constexpr int es = KV == KV_F32 ? 4 : (KV == KV_BF16 ? 2 : 1);
};

struct AttnArgs {
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* slot_block;
  int N, H, v_ld;
  const void* q;
  int n_q, q_pos0, q_block0, q_block_len;
  float bias_log2;   // cache_bias * log2(e)
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  float* lse;
  float* part_o;    // [splits][n_q][H][d] when split
  float* part_lse;  // [splits][H][n_q]
  int n_qt, n_splits, tiles_per_split, n_tiles;
  int remap;    // blockIdx -> work item remap keeps a head's tiles on one XCD
  int n_items;  // workgroups launched
  int use_rope;
  RopeTable rope;
  const int32_t* q_block_ids;  // [n_q] block per query, or null: q_block0 + i / q_block_len
  int same_block;              // mask: visible iff slot block == query block (no bias)
};

// LDS geometry of one tile buffer (K rows, then V^T rows).
template <int KV, int D>
struct Tile {
  static constexpr int es = KvT<KV>::es;
  static constexpr int k_row = D * es;  // bytes per K row
  static constexpr int k_cpr = k_row / 16;
  static constexpr int v_row = kKT * es;  // bytes per V^T row
  static constexpr int v_cpr = v_row / 16;
  static constexpr int k_off = 0;
  static constexpr int v_off = kKT * k_row;
  static constexpr int bytes = v_off + D * v_row;
  static constexpr int k_instr = kKT * k_cpr / (kQSub * kWave);  // 16-byte DMA per wave
  static constexpr int v_instr = D * v_cpr / (kQSub * kWave);
  static constexpr int dma_instr = k_instr + v_instr;
  static_assert(kKT * k_cpr % (kQSub * kWave) == 0 && D * v_cpr % (kQSub * kWave) == 0, "tile split");
};

// Per-slot factors of one tile for one key half, written once by one wave of
// the half a step before the tile is used (words, 64 per array):
//   A  = c s_k            the logit is A * S' with S' the QK accumulator
//   C  = log2(s_v) / A    accumulator start, so that A * S' = y0 + log2 s_v
//   iv = 1 / s_v          weight of P~ in the running sum
//   kb = block id of the slot (-1: empty)
// and a summary {any slot valid, all valid, min and max block over valid
// slots} from which every wave classifies the tile with scalar tests.
constexpr int kFacA = 0, kFacC = kKT, kFacIv = 2 * kKT, kFacKb = 3 * kKT;
constexpr int kFacSum = 4 * kKT;
constexpr int kFacWords = 4 * kKT + 4;
constexpr float kMinA = 0x1p-90f;  // floor of A, so that C stays finite

// Slot metadata of one tile moves in one 1 KB load: 16-byte chunks 0..15
// are k_scale, 16..31 v_scale, 32..47 slot_block (FP8); without scales every
// group of 16 chunks is slot_block.  Chunks 48..63 repeat slot_block, so
// that all 64 lanes load.
constexpr int kMetaWords = 256;
constexpr int kMetaKs = 0, kMetaVs = 64, kMetaKb = 128;

template <int KV, int D>
struct Stages {
  // Double buffering; each stage holds kps tiles per key half (two when they
  // fit) and their factor tables.
  static constexpr int need(int kps) {
    return 2 * kHalves * kps * (Tile<KV, D>::bytes + kFacWords * 4 + kMetaWords * 4) + 256;
  }
  static constexpr int kps = need(2) <= 160 * 1024 ? 2 : 1;
  static_assert(need(kps) <= 160 * 1024, "LDS budget");
};

// Slot (row of the K tile) that lane row m of M-block mb feeds into the QK
// MFMA, so that accumulator element i of lane group g is slot 32g + 16mb + i.
__device__ __forceinline__ int k_perm(int mb, int m) {
  return 32 * ((m >> 2) & 1) + 16 * mb + 4 * (m >> 3) + (m & 3);
}

// XOR swizzles of 16-byte chunks against LDS bank conflicts, chosen by
// measuring the conflict counter for each read pattern below: the K reads
// take one chunk column of the slots k_perm(mb, 0..31), the V^T reads one
// chunk column of 32 consecutive rows d.
template <int KV, int D>
__device__ __forceinline__ int k_swz(int slot) {
  constexpr int cpr = Tile<KV, D>::k_cpr;
  if constexpr (cpr == 4) return (slot ^ (slot >> 2)) & 3;   // 64-byte rows
  else if constexpr (cpr == 8) return (slot >> 1) & 7;      // 128-byte rows
  else return slot & 15;                                    // 256-byte rows
}
template <int KV, int D>
__device__ __forceinline__ int v_swz(int d) {
  constexpr int cpr = Tile<KV, D>::v_cpr;
  if constexpr (cpr == 4) return (d ^ (d >> 2)) & 3;
  else if constexpr (cpr == 8) return (d >> 1) & 7;
  else return d & 15;
}
template <int KV, int D>
__device__ __forceinline__ int k_addr(int slot, int c) {
  return slot * Tile<KV, D>::k_row + ((c ^ k_swz<KV, D>(slot)) << 4);
}
template <int KV, int D>
__device__ __forceinline__ int v_addr(int d, int c) {
  return Tile<KV, D>::v_off + d * Tile<KV, D>::v_row + ((c ^ v_swz<KV, D>(d)) << 4);
}

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_wave_base) {
  // address-space conversions: generic -> global (1) and generic -> LDS (3)
  __builtin_amdgcn_global_load_lds((glb_void*)(g), (lds_void*)(lds_wave_base), 16, 0, 0);
}

// The same load from a buffer: 32-bit lane offset plus a scalar offset, no
// 64-bit vector address per load (the tile loads use this form; a raw buffer
// returns zeros past its end).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff,
                                          uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_wave_base), 16, static_cast<int>(off),
                                           static_cast<int>(soff), 0, 0);
}

// Direct-to-LDS loads of one tile for one key half.  Every wave of the half
// moves whole 1 KB blocks (64 lanes x 16 bytes, contiguous in LDS); each lane
// picks the global chunk that belongs at its LDS position.  The lane's byte
// offsets do not depend on the tile, so they are computed once: a tile load
// is a uniform base address plus these offsets.  K rows are padded to v_ld
// slots per head, so a tile never reads past its head; padding slots hold
// zeros and block -1.
template <int KV, int D>
struct DmaPlan {
  uint32_t k[Tile<KV, D>::k_instr];  // from the tile's first K row
  uint32_t v[Tile<KV, D>::v_instr];  // from V^T[h][0][first slot of the tile]
  const uint8_t* meta;               // this lane's metadata chunk of tile 0
  __amdgpu_buffer_rsrc_t k_rsrc;     // this head's K rows [v_ld][D]
  __amdgpu_buffer_rsrc_t v_rsrc;     // this head's V^T rows [D][v_ld]
};


template <int KV, int D>
__device__ __forceinline__ DmaPlan<KV, D> dma_plan(const AttnArgs& a, int h, int wq, int lane) {
  using T = Tile<KV, D>;
  DmaPlan<KV, D> pl;
  const int which = KV == KV_FP8 ? min(lane >> 4, 2) : 2;
  const int j = (lane & 15) * 4;
  const size_t hs = static_cast<size_t>(h) * a.v_ld + j;
  pl.meta = which == 0 ? reinterpret_cast<const uint8_t*>(a.k_scale + hs)
            : which == 1 ? reinterpret_cast<const uint8_t*>(a.v_scale + hs)
                         : reinterpret_cast<const uint8_t*>(a.slot_block + j);
  pl.k_rsrc = make_rsrc(a.k + static_cast<size_t>(h) * a.v_ld * T::k_row, static_cast<uint32_t>(a.v_ld) * T::k_row);
  pl.v_rsrc = make_rsrc(a.v + static_cast<size_t>(h) * D * a.v_ld * T::es, static_cast<uint32_t>(D * a.v_ld * T::es));
#pragma unroll
  for (int j = 0; j < T::k_instr; ++j) {
    const int p = (wq * T::k_instr + j) * kWave + lane;  // LDS chunk index
    const int r = p / T::k_cpr, cp = p % T::k_cpr;
    pl.k[j] = static_cast<uint32_t>(r * T::k_row + ((cp ^ k_swz<KV, D>(r)) << 4));
  }
#pragma unroll
  for (int j = 0; j < T::v_instr; ++j) {
    const int p = (wq * T::v_instr + j) * kWave + lane;
    const int d = p / T::v_cpr, cp = p % T::v_cpr;
    pl.v[j] = static_cast<uint32_t>(d * a.v_ld * T::es + ((cp ^ v_swz<KV, D>(d)) << 4));
  }
  return pl;
}

// The j-th of this wave's dma_instr loads of one tile (K blocks first).
template <int KV, int D>
__device__ __forceinline__ void issue_part(const AttnArgs& a, const DmaPlan<KV, D>& pl, int h, int tile,
                                           uint8_t* buf, int wq, int j) {
  using T = Tile<KV, D>;
  if (j < T::k_instr) {
    dma16_buf(pl.k_rsrc, pl.k[j], static_cast<uint32_t>(tile * kKT * T::k_row),
              buf + T::k_off + (wq * T::k_instr + j) * 1024);
  } else {
    const int jv = j - T::k_instr;
    dma16_buf(pl.v_rsrc, pl.v[jv], static_cast<uint32_t>(tile * kKT * T::es),
              buf + T::v_off + (wq * T::v_instr + jv) * 1024);
  }
}

// s_waitcnt vmcnt(N) as a real instruction (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maxima),
// so that the compiler's own wait insertion accounts for it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding load, including tiles still in flight.
// Callers wait for exactly what must be visible first.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Q operand registers of one lane (query n = lane % 32, group g = lane / 32).
template <int KV, int D>
struct QFrag;
template <int D>
struct QFrag<KV_FP8, D> {
  v8i q[D / 64];
};
template <int D>
struct QFrag<KV_BF16, D> {
  v8bf q[D / 16];
};
template <int D>
struct QFrag<KV_F32, D> {
  float q[D / 2];
};

// d index of element e (0..D/2-1) held by lane group g in the Q operand.
template <int KV, int D>
__device__ __forceinline__ int q_dim(int g, int e) {
  if constexpr (KV == KV_FP8) return (e / 32) * 64 + 32 * g + (e % 32);
  else if constexpr (KV == KV_BF16) return (e / 8) * 16 + 8 * g + (e % 8);
  else return 2 * e + g;
}

// Four floats to four e4m3 codes written over `old`; both halves of the word
// are replaced, so passing the word's previous value avoids clearing it.
__device__ __forceinline__ int cvt_fp8x4_over(float a, float b, float c, float d, int old) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Reduction over the 64 lanes without LDS: quad permutes and row rotations
// (DPP) inside each row of 16 lanes, then row-pair and half swaps.
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

// GEN: per-query block ids and the same-block mask (rc_chunk_attention_ex);
// without it the kernel is the plain block-causal one.
template <int KV, int D, bool GEN>
__global__ __launch_bounds__(kThreads) void chunk_attn_kernel(AttnArgs a) {
  using T = Tile<KV, D>;
  constexpr int KPS = Stages<KV, D>::kps;
  // One array per pipeline stage (kps tiles for each key half).  Separate
  // objects let the compiler see that reading one stage does not depend on
  // the loads still landing in the other, so it adds no waits of its own.
  constexpr int kStageBytes = kHalves * KPS * T::bytes;
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  // Factor tables of the two stages: [half][kps][kFacWords].
  __shared__ __attribute__((aligned(16))) float fac0[kHalves * KPS * kFacWords];
  __shared__ __attribute__((aligned(16))) float fac1[kHalves * KPS * kFacWords];
  // Slot metadata, two steps ahead: [half][kps][kMetaWords] per array.
  __shared__ __attribute__((aligned(16))) float meta0[kHalves * KPS * kMetaWords];
  __shared__ __attribute__((aligned(16))) float meta1[kHalves * KPS * kMetaWords];
  __shared__ float red[kWaves];

  // Every argument used before the first loads is read here in one batch of
  // scalar loads; the empty asm keeps them from being spread over the
  // dependent steps below (one argument round trip instead of several).
  asm volatile("" ::"s"(a.n_qt), "s"(a.n_splits), "s"(a.tiles_per_split), "s"(a.n_tiles), "s"(a.remap),
               "s"(a.n_items), "s"(a.v_ld), "s"(a.H), "s"(a.n_q), "s"(a.k), "s"(a.v), "s"(a.q),
               "s"(a.slot_block), "s"(a.k_scale), "s"(a.v_scale));
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: kept in SGPRs
  const int kh = wave / kQSub;  // key half
  const int wq = wave % kQSub;  // query sub-tile (and wave index inside the half)
  const int n = lane & 31;
  const int g = lane >> 5;

  // ---- work item
  int item = blockIdx.x;
  if (a.remap) item = (item % 8) * (a.n_items / 8) + item / 8;
  const int qt = item % a.n_qt;
  const int hs = item / a.n_qt;
  const int split = hs % a.n_splits;
  const int h = hs / a.n_splits;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.n_tiles, t_begin + a.tiles_per_split);
  // local tile li of this half is tile t_begin + 2 li + kh; a step covers
  // local tiles KPS*step .. KPS*step + KPS-1
  const int n_local = (max(t_end - t_begin, 0) + 1) / 2;
  const int n_steps = (n_local + KPS - 1) / KPS;
  auto tile_of = [&](int li) { return t_begin + 2 * li + kh; };
  auto has_tile = [&](int li) { return li < n_local && tile_of(li) < t_end; };
  // a tile that exists, reloaded where a load has no tile of its own
  const int t_safe = min(t_begin, a.n_tiles - 1);
  auto tile_buf = [&](uint8_t* stage, int kk) { return stage + (kh * KPS + kk) * T::bytes; };
  auto fac_tbl = [&](float* ftab, int kk) { return ftab + (kh * KPS + kk) * kFacWords; };
  const DmaPlan<KV, D> plan = dma_plan<KV, D>(a, h, wq, lane);
  // Every step issues KPS tiles' loads for every wave (past the end a valid
  // tile is reloaded into a slot nobody reads), so wait counts are uniform.
  auto issue_j = [&](uint8_t* stage, int st, int kk, int j) {
    const int li = st * KPS + kk;
    issue_part<KV, D>(a, plan, h, has_tile(li) ? tile_of(li) : t_safe, tile_buf(stage, kk), wq, j);
  };
  auto issue = [&](uint8_t* stage, int st, int kk) {
#pragma unroll
    for (int j = 0; j < T::dma_instr; ++j) issue_j(stage, st, kk, j);
  };

  // ---- queries of this lane
  const int q_base = qt * kQT;
  const int iq = wq * kQW + n;
  const int qi = q_base + iq;
  const bool q_ok = qi < a.n_q;
  const int wave_q0 = q_base + wq * kQW;
  const bool wave_active = wave_q0 < a.n_q;
  const int wave_q1 = max(min(wave_q0 + kQW, a.n_q) - 1, wave_q0);
  int qb_lo = a.q_block0 + wave_q0 / a.q_block_len;
  int qb_hi = a.q_block0 + wave_q1 / a.q_block_len;
  int my_qb = a.q_block0 + (q_ok ? qi : wave_q0) / a.q_block_len;
  if (GEN && a.q_block_ids) {  // explicit blocks: the wave's range from a reduction
    my_qb = a.q_block_ids[q_ok ? qi : min(wave_q0, a.n_q - 1)];
    qb_lo = __builtin_amdgcn_readfirstlane(wave_minmax_i32<false>(my_qb));
    qb_hi = __builtin_amdgcn_readfirstlane(wave_minmax_i32<true>(my_qb));
  }
  const bool same_block = GEN && a.same_block != 0;
  const int lo_qb = same_block ? my_qb : 0;  // lowest visible block (empty slots hold -1)

  // ---- slot metadata for the factor tables.  Wave f = wq of key half 0
  //      builds table f (tile f % KPS of half f / KPS) of every step, from
  //      metadata it loads into LDS two steps ahead (past the end a valid
  //      tile is reloaded, so every factor wave issues the same loads).  The
  //      work sits in half 0 because its waves are the older ones on each
  //      SIMD, which issue first and otherwise wait at the step barrier.
  const int fac_id = wq;
  const bool fac_wave = kh == 0 && fac_id < kHalves * KPS;
  const int fh = fac_id / KPS, fk = fac_id % KPS;
  auto meta_issue = [&](float* mbuf, int st) {
    const int li = st * KPS + fk;
    const int tf = t_begin + 2 * li + fh;
    const int tile = li < n_local && tf < t_end ? tf : t_safe;
    dma16(plan.meta + tile * (kKT * 4), reinterpret_cast<uint8_t*>(mbuf + fac_id * kMetaWords));
  };
  if (fac_wave) {
    meta_issue(meta0, 0);
    meta_issue(meta1, 1);
  }

  // ---- raw Q of this lane.  Lane group g holds half of the query's d values
  //      in runs of even length (both members of every RoPE pair) for
  //      FP8/BF16; for F32 every pair (2e, 2e+1).  The first step's tiles
  //      are issued after these loads, so waiting for Q does not wait for
  //      them (they go out even for an empty key range, from a valid tile).
  constexpr int kQRaw = KV == KV_F32 ? D / 4 : D / 16;  // 16-byte loads per lane
  v4u qraw[kQRaw];
  {
    const size_t qrow = (static_cast<size_t>(q_ok ? qi : 0) * a.H + h) * D;
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) + qrow * (KV == KV_F32 ? 4 : 2);
#pragma unroll
    for (int r = 0; r < kQRaw; ++r) {
      int byte_off;
      if constexpr (KV == KV_FP8) byte_off = ((r / 4) * 64 + 32 * g) * 2 + (r % 4) * 16;
      else if constexpr (KV == KV_BF16) byte_off = (r * 16 + 8 * g) * 2;
      else byte_off = r * 16;
      qraw[r] = *reinterpret_cast<const v4u*>(qb + byte_off);
    }
  }
#pragma unroll
  for (int kk = 0; kk < KPS; ++kk) issue(st0, 0, kk);
  // keep the work on Q below these loads, so that waiting for Q does not
  // hold back their issue
  __builtin_amdgcn_sched_barrier(0);

  // ---- Q: rotate, (quantise) into MFMA operand registers
  QFrag<KV, D> qf;
  float c_mul = a.scale_log2;  // y = c_mul * s_k * S + ...
  const bool use_rope = a.use_rope != 0;
  const long long qpos = static_cast<long long>(a.q_pos0) + qi;
  {
    float x[D / 2];
    if constexpr (KV == KV_F32) {
      // qraw holds (q[4r], q[4r+1], q[4r+2], q[4r+3]); element e is d = 2e + g
#pragma unroll
      for (int e = 0; e < D / 2; ++e) {
        const v4u w = qraw[e / 2];
        const float x0 = __uint_as_float((e & 1) ? w.z : w.x);
        const float x1 = __uint_as_float((e & 1) ? w.w : w.y);
        float y0 = x0, y1 = x1;
        if (use_rope) {
          float c, sn;
          rope_cs_hw(a.rope.rev[e], qpos, &c, &sn);
          y0 = x0 * c - x1 * sn;
          y1 = x0 * sn + x1 * c;
        }
        x[e] = q_ok ? (g ? y1 : y0) : 0.f;
      }
    } else {
      // qraw word k holds bf16 elements (2k, 2k+1) of this lane's run order
#pragma unroll
      for (int e = 0; e < D / 2; e += 2) {
        const uint32_t w = qraw[e / 8][(e / 2) % 4];
        const float x0 = __uint_as_float(w << 16);
        const float x1 = __uint_as_float(w & 0xFFFF0000u);
        float y0 = x0, y1 = x1;
        if (use_rope) {
          // pair j = q_dim(g, e) / 2: one of two wave-uniform frequencies
          const int j0 = q_dim<KV, D>(0, e) >> 1, j1 = q_dim<KV, D>(1, e) >> 1;
          const double rev0 = a.rope.rev[j0], rev1 = a.rope.rev[j1];
          float c, sn;
          rope_cs_hw(g ? rev1 : rev0, qpos, &c, &sn);
          y0 = x0 * c - x1 * sn;
          y1 = x0 * sn + x1 * c;
        }
        x[e] = q_ok ? y0 : 0.f;
        x[e + 1] = q_ok ? y1 : 0.f;
      }
    }
    if constexpr (KV == KV_FP8) {
      // one scale for the workgroup's 128 queries: s_q = max|q| / 448
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < D / 2; ++e) am = fmaxf(am, fabsf(x[e]));
      am = group_max<kWave>(am);
      if (lane == 0) red[wave] = am;
      wait_lgkm0();
      bare_barrier();
      am = red[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) am = fmaxf(am, red[w]);
      const float sq = am > 0.f ? am / 448.f : 1.f;
      const float iq8 = am > 0.f ? 448.f / am : 0.f;
      c_mul = a.scale_log2 * sq;
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int e = ks * 32 + 4 * w;
          qf.q[ks][w] =
              static_cast<int>(cvt_fp8x4(x[e] * iq8, x[e + 1] * iq8, x[e + 2] * iq8, x[e + 3] * iq8));
        }
      }
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf.q[ks][e] = static_cast<__bf16>(x[ks * 8 + e]);
    } else {
#pragma unroll
      for (int e = 0; e < D / 2; ++e) qf.q[e] = x[e];
    }
  }

  // ---- accumulators
  v16f o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = v16f{};
  float m_run = -INFINITY;  // stabiliser (log2 units)
  float msub = 0.f;         // m_run, or 0 while it is -inf: logits are held as y - msub
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's partial sums of p
  v8i pb = {};  // FP8 P^T operand, rewritten by every tile

  // ---- factor tables: the table of the half's tile kk of the next step is
  //      written by wave kk of the half (fac_write, below) from the slot
  //      metadata loaded here at the start of the current step.
  auto fac_write = [&](const float* mbuf, float* tbl) {
    const float* mt = mbuf + fac_id * kMetaWords;
    const int kb = reinterpret_cast<const int32_t*>(mt)[kMetaKb + lane];
    const bool kval = kb != -1;
    float A = c_mul, lv = 0.f, ivf = 1.f;
    if constexpr (KV == KV_FP8) {
      const float vs = fmaxf(mt[kMetaVs + lane], kMinVScale);
      A = fmaxf(c_mul * mt[kMetaKs + lane], kMinA);
      lv = __builtin_amdgcn_logf(vs);
      ivf = __builtin_amdgcn_rcpf(vs);
    }
    const float rA = __builtin_amdgcn_rcpf(A);
    tbl[kFacA + lane] = A;
    tbl[kFacC + lane] = lv * rA;
    tbl[kFacIv + lane] = ivf;
    reinterpret_cast<int32_t*>(tbl)[kFacKb + lane] = kb;
    const uint64_t vb = __ballot(kval);
    const int kmin = wave_minmax_i32<false>(kval ? kb : INT32_MAX);
    const int kmax = wave_minmax_i32<true>(kval ? kb : INT32_MIN);
    if (lane == 0)
      *reinterpret_cast<v4i*>(tbl + kFacSum) = v4i{vb != 0ull ? 1 : 0, vb == ~0ull ? 1 : 0, kmin, kmax};
  };
  // Wave-uniform tile class from the summary: vis (some query of the wave
  // sees some slot), fast (every slot visible to every query with one bias
  // value) and hist (fast, and every slot takes the bias).
  auto classify = [&](const float* tbl, bool& vis, bool& fast, bool& hist) {
    const v4i sm = *reinterpret_cast<const v4i*>(tbl + kFacSum);
    const int any = __builtin_amdgcn_readfirstlane(sm.x);
    const int all = __builtin_amdgcn_readfirstlane(sm.y);
    const int kmin = __builtin_amdgcn_readfirstlane(sm.z);
    const int kmax = __builtin_amdgcn_readfirstlane(sm.w);
    const bool all_same = qb_lo == qb_hi && all && kmin == qb_lo && kmax == qb_lo;
    if (GEN && same_block) {  // slots of the query's own block only, never biased
      vis = any && kmin <= qb_hi && kmax >= qb_lo;
      fast = all_same;
      hist = false;
      return;
    }
    vis = any && kmin <= qb_hi;
    const bool all_vis = all && kmax <= qb_lo;
    const bool all_hist = all && kmax < qb_lo;
    fast = all_vis && (all_hist || all_same || a.bias_log2 == 0.f);
    hist = fast && all_hist;
  };

  // S'^T = K Q^T + C: accumulator element i of lane group g is slot
  // 32g + 16mb + i, and starts at that slot's C so that A * S' = y.
  auto qk = [&](const uint8_t* buf, const float* ctab, v16f (&s)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float* cf = ctab + 32 * g + 16 * mb;
      const v4f c0 = *reinterpret_cast<const v4f*>(cf), c1 = *reinterpret_cast<const v4f*>(cf + 4);
      const v4f c2 = *reinterpret_cast<const v4f*>(cf + 8), c3 = *reinterpret_cast<const v4f*>(cf + 12);
      s[mb] = v16f{c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w,
                   c2.x, c2.y, c2.z, c2.w, c3.x, c3.y, c3.z, c3.w};
      const int slot = k_perm(mb, n);
      if constexpr (KV == KV_FP8) {
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
          const int c0i = 4 * ks + 2 * g;
          const v4i lo = *reinterpret_cast<const v4i*>(buf + k_addr<KV, D>(slot, c0i));
          const v4i hi = *reinterpret_cast<const v4i*>(buf + k_addr<KV, D>(slot, c0i + 1));
          const v8i av = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          s[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf.q[ks], s[mb], 0, 0, 0, 0, 0, 0);
        }
      } else if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const v8bf av = *reinterpret_cast<const v8bf*>(buf + k_addr<KV, D>(slot, 2 * ks + g));
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf.q[ks], s[mb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) {
          const int dd = 2 * ks + g;
          const float av = *reinterpret_cast<const float*>(buf + k_addr<KV, D>(slot, dd >> 2) + (dd & 3) * 4);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, qf.q[ks], s[mb], 0, 0, 0);
        }
      }
    }
  };

  // Softmax update and O^T += V^T P^T for one tile.
  auto smpv = [&](const uint8_t* buf, const float* wf, v16f (&s)[2], bool fast, bool hist) {
    // -- z = A S' (+ bias) - msub = y - msub, masked to -inf.  A fast tile
    //    takes the bias on every slot or on none.
    const float negm = -msub;
    if (fast) {
      const float zadd = hist ? negm + a.bias_log2 : negm;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const v4f af = *reinterpret_cast<const v4f*>(wf + 32 * g + 16 * mb + 4 * qq);
          s[mb][4 * qq + 0] = fmaf(s[mb][4 * qq + 0], af.x, zadd);
          s[mb][4 * qq + 1] = fmaf(s[mb][4 * qq + 1], af.y, zadd);
          s[mb][4 * qq + 2] = fmaf(s[mb][4 * qq + 2], af.z, zadd);
          s[mb][4 * qq + 3] = fmaf(s[mb][4 * qq + 3], af.w, zadd);
        }
    } else {
      const int32_t* kbs = reinterpret_cast<const int32_t*>(wf + kFacKb);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int slot0 = 32 * g + 16 * mb + 4 * qq;
          const v4f af = *reinterpret_cast<const v4f*>(wf + slot0);
          const v4i kb4 = *reinterpret_cast<const v4i*>(kbs + slot0);
          const float afa[4] = {af.x, af.y, af.z, af.w};
          const int kba[4] = {kb4.x, kb4.y, kb4.z, kb4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // visible iff lo_qb <= block <= my_qb (lo_qb = 0, or the query's
            // own block for the same-block mask, whose bias is zero)
            const int kb = kba[r];
            const int cls = !GEN ? visibility_class(kb, my_qb)
                                 : (kb < lo_qb || kb > my_qb) ? kVisNone : (kb < my_qb ? kVisBias : kVisPlain);
            float z = fmaf(s[mb][4 * qq + r], afa[r], negm);
            z = cls == kVisBias ? z + a.bias_log2 : z;
            s[mb][4 * qq + r] = cls == kVisNone ? -INFINITY : z;
          }
        }
    }
    // -- tile maximum of this query (both lane groups)
    float tmax;
    {
      // four independent chains of three-input maxima over 8 values each
      float c4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const v16f& v = s[k >> 1];
        const int o = 8 * (k & 1);
        float t = fmaxf(fmaxf(v[o], v[o + 1]), v[o + 2]);
        t = fmaxf(fmaxf(t, v[o + 3]), v[o + 4]);
        t = fmaxf(fmaxf(t, v[o + 5]), v[o + 6]);
        c4[k] = fmaxf(t, v[o + 7]);
      }
      tmax = fmaxf(fmaxf(fmaxf(c4[0], c4[1]), c4[2]), c4[3]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // -- raise the stabiliser only when the tile maximum passes it by tau
    if (__ballot(tmax + msub > m_run + kTau) != 0ull) {
      const float m_new = fmaxf(m_run, tmax + msub);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 4; ++r) l_part[r] *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b) o[b] *= alpha;
      const float shift = m_new == -INFINITY ? 0.f : m_new - msub;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[mb] -= shift;
      m_run = m_new;
      msub = m_new == -INFINITY ? 0.f : m_new;
    }

    // -- P~ = 2^z; l += P~ / s_v
    const float* ivfp = wf + kFacIv;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const v4f iv = *reinterpret_cast<const v4f*>(ivfp + 32 * g + 16 * mb + 4 * qq);
        const float iva[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[mb][4 * qq + r]);
          s[mb][4 * qq + r] = p;
          l_part[r] = fmaf(p, iva[r], l_part[r]);
        }
      }
    }

    // -- O^T += V^T P^T (reduction index: slot 32g + j of the tile)
    if constexpr (KV == KV_FP8) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          pb[4 * mb + qq] = cvt_fp8x4_over(s[mb][4 * qq], s[mb][4 * qq + 1], s[mb][4 * qq + 2],
                                           s[mb][4 * qq + 3], pb[4 * mb + qq]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + n;
        const v4i lo = *reinterpret_cast<const v4i*>(buf + v_addr<KV, D>(d, 2 * g));
        const v4i hi = *reinterpret_cast<const v4i*>(buf + v_addr<KV, D>(d, 2 * g + 1));
        const v8i av = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, o[db], 0, 0, 0, 0, 0, 0);
      }
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        v8bf pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[st >> 1][8 * (st & 1) + e]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = 32 * db + n;
          const v8bf av = *reinterpret_cast<const v8bf*>(buf + v_addr<KV, D>(d, 4 * g + st));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[db], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int slot = 32 * g + 16 * mb + 4 * e4;  // one 16-byte chunk: slots slot .. slot + 3
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + n;
            const v4f av = *reinterpret_cast<const v4f*>(buf + v_addr<KV, D>(d, slot >> 2));
#pragma unroll
            for (int k = 0; k < 4; ++k)
              o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[k], s[mb][4 * e4 + k], o[db], 0, 0, 0);
          }
        }
      }
    }
  };

  // One pipeline step: the KPS tiles of stage `cur` are computed while the
  // next step's tiles are loaded into `nxt` and the factor waves fill the
  // next step's tables.  A wave issues its loads of next-step tile kk right
  // after the QK MFMAs of current tile kk, so that the issue (which stalls
  // while the load queue is busy) overlaps matrix work.
  auto step = [&](uint8_t* cur, uint8_t* nxt, float* fcur, float* fnxt, float* mcur, float* mnxt, int st) {
    wait_vm<0>();    // this wave's loads of this step have landed
    wait_lgkm0();    // and its table writes are done
    bare_barrier();  // every wave's: visible to all; every wave is done with `nxt`
    const bool more = st + 1 < n_steps;
    if (fac_wave && st + 2 < n_steps) meta_issue(mcur, st + 2);
    if (!wave_active) {
      if (more) {
#pragma unroll
        for (int kk = 0; kk < KPS; ++kk) issue(nxt, st + 1, kk);
      }
    } else {
      bool vis[KPS], fast[KPS], hist[KPS];
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) {
        classify(fac_tbl(fcur, kk), vis[kk], fast[kk], hist[kk]);
        vis[kk] = vis[kk] && has_tile(st * KPS + kk);
      }
#pragma unroll
      for (int kk = 0; kk < KPS; ++kk) {
        const float* tbl = fac_tbl(fcur, kk);
        // QK runs even for a tile the wave cannot see (its result is then
        // unused): its LDS reads then overlap those of the tile summary.
        v16f sc[2];
        qk(tile_buf(cur, kk), tbl + kFacC, sc);
        if (more) issue(nxt, st + 1, kk);
        if (vis[kk]) smpv(tile_buf(cur, kk), tbl, sc, fast[kk], hist[kk]);
      }
    }
    if (fac_wave && more) fac_write(mnxt, fnxt + fac_id * kFacWords);
  };
  if (n_steps > 0 && fac_wave) fac_write(meta0, fac0 + fac_id * kFacWords);
  for (int st = 0; st < n_steps; st += 2) {
    step(st0, st1, fac0, fac1, meta0, meta1, st);
    if (st + 1 < n_steps) step(st1, st0, fac1, fac0, meta1, meta0, st + 1);
  }

  // ---- merge the two key halves of every query sub-tile through LDS
  float l_sum = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  __syncthreads();  // all tiles consumed; stage buffers are free
  static_assert(2 * kWave * (D / 2 + 2) * 4 <= kStageBytes, "merge buffer");
  float* xch = (wq < 2 ? reinterpret_cast<float*>(st0) : reinterpret_cast<float*>(st1)) +
               ((wq & 1) * kWave + lane) * (D / 2 + 2);
  if (kh == 1) {
    xch[0] = m_run;
    xch[1] = l_sum;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) xch[2 + 16 * b + e] = o[b][e];
  }
  __syncthreads();
  if (kh == 1 || !wave_active) return;
  {
    const float m1 = xch[0], l1 = xch[1];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_sum = a0 * l_sum + a1 * l1;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][e] = a0 * o[b][e] + a1 * xch[2 + 16 * b + e];
    m_run = mm;
  }

  // ---- epilogue
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_sum), __float_as_uint(l_sum), false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool any = m_run != -INFINITY && l_tot > 0.f;
  const float oscale = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!q_ok) return;
  if (a.n_splits == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * g;
        const size_t off = (static_cast<size_t>(qi) * a.H + h) * D + d;
        const float r0 = o[db][4 * qq] * oscale, r1 = o[db][4 * qq + 1] * oscale;
        const float r2 = o[db][4 * qq + 2] * oscale, r3 = o[db][4 * qq + 3] * oscale;
        if constexpr (KV == KV_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = make_float4(r0, r1, r2, r3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
              make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
        }
      }
    }
    if (a.lse && g == 0) a.lse[static_cast<size_t>(h) * a.n_q + qi] = lse_v;
  } else {
    float* po = a.part_o + ((static_cast<size_t>(split) * a.n_q + qi) * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * g;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(o[db][4 * qq] * oscale, o[db][4 * qq + 1] * oscale, o[db][4 * qq + 2] * oscale,
                        o[db][4 * qq + 3] * oscale);
      }
    if (g == 0) a.part_lse[(static_cast<size_t>(split) * a.H + h) * a.n_q + qi] = lse_v;
  }
}

// Merge split partials (each normalised by its own sum) in fixed split order:
// out = sum_s exp(lse_s - LSE) o_s,  LSE = ln sum_s exp(lse_s).
template <int KV, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* part_o, const float* part_lse,
                                                      int n_splits, int n_q, int H, void* out,
                                                      float* lse) {
  const int row = blockIdx.x * (256 / 32) + threadIdx.x / 32;  // (query, head) row
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
  for (int e = 0; e < D / 32; ++e) {
    const size_t off = static_cast<size_t>(row) * D + lane + 32 * e;
    if constexpr (KV == KV_F32) static_cast<float*>(out)[off] = acc[e] * inv;
    else static_cast<uint16_t*>(out)[off] = f32_to_bf16(acc[e] * inv);
  }
  if (lse && lane == 0) lse[static_cast<size_t>(h) * n_q + qi] = mx == -INFINITY ? -INFINITY : mx + logf(wsum);
}

__global__ __launch_bounds__(256) void visibility_kernel(const int32_t* slot_block, int N, int n_q,
                                                         int q_block0, int q_block_len, uint8_t* mask) {
  const size_t total = static_cast<size_t>(n_q) * N;
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total; e += gridDim.x * 256ull) {
    const int qi = static_cast<int>(e / N), s = static_cast<int>(e % N);
    const int qb = q_block0 + qi / q_block_len;
    mask[e] = static_cast<uint8_t>(visibility_class(slot_block[s], qb));
  }
}

template <int KV, int D>
hipError_t attn_impl(const RingView& r, const AttnCall& c, int splits, hipStream_t s) {
  AttnArgs a{};
  a.k = static_cast<const uint8_t*>(r.k);
  a.v = static_cast<const uint8_t*>(r.v);
  a.k_scale = r.k_scale;
  a.v_scale = r.v_scale;
  a.slot_block = r.slot_block;
  a.N = r.N;
  a.H = r.H;
  a.v_ld = r.v_ld;
  a.q = c.q;
  a.n_q = c.n_q;
  a.q_pos0 = c.q_pos0;
  a.q_block0 = c.q_block0;
  a.q_block_len = c.q_block_len;
  a.q_block_ids = c.q_block_ids;
  a.same_block = c.same_block;
  const float sigma = c.softmax_scale != 0.f ? c.softmax_scale : 1.f / std::sqrt(static_cast<float>(r.d));
  a.scale_log2 = sigma * kLog2e;
  a.bias_log2 = c.same_block ? 0.f : c.cache_bias * kLog2e;  // the same-block mask has no earlier blocks
  a.out = c.out;
  a.lse = c.lse;
  a.n_qt = (c.n_q + kQT - 1) / kQT;
  a.n_tiles = (r.N + kKT - 1) / kKT;
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
  if (a.q_block_ids || a.same_block)
    hipLaunchKernelGGL((chunk_attn_kernel<KV, D, true>), dim3(total), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_attn_kernel<KV, D, false>), dim3(total), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int rows = c.n_q * r.H;
  hipLaunchKernelGGL((combine_kernel<KV, D>), dim3((rows + 7) / 8), dim3(256), 0, s, a.part_o, a.part_lse,
                     splits, c.n_q, r.H, c.out, c.lse);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int kv, int d) { return !(kv == KV_F32 && d == 128); }

int attention_splits(const RingView& r, int n_q) {
  if (r.kv == KV_FP8) return fp8_attention_splits(r, n_q);
  const int n_qt = (n_q + kQT - 1) / kQT;
  const int n_tiles = (r.N + kKT - 1) / kKT;
  const int items = n_qt * r.H;
  // Split the key range only when the grid is far below one workgroup per CU;
  // each split keeps at least 4 tiles (2 per key half).
  int splits = 1;
  while (items * splits * 2 <= 256 && (splits * 2) * 4 <= n_tiles) splits *= 2;
  return splits;
}

size_t attention_workspace_bytes(const RingView& r, int n_q) {
  const int splits = attention_splits(r, n_q);
  if (splits == 1) return 0;
  return static_cast<size_t>(splits) * n_q * r.H * (r.d + 1) * sizeof(float);
}

hipError_t launch_chunk_attention(const RingView& r, const AttnCall& c, hipStream_t s) {
  int splits = attention_splits(r, c.n_q);
  if (splits > 1 && (c.workspace == nullptr || c.workspace_bytes < attention_workspace_bytes(r, c.n_q)))
    splits = 1;
  if (r.kv == KV_FP8) return launch_fp8_attention(r, c, splits, s);
  switch (r.kv * 1000 + r.d) {
    case KV_BF16 * 1000 + 128: return attn_impl<KV_BF16, 128>(r, c, splits, s);
    case KV_BF16 * 1000 + 64: return attn_impl<KV_BF16, 64>(r, c, splits, s);
    case KV_F32 * 1000 + 64: return attn_impl<KV_F32, 64>(r, c, splits, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_debug_visibility(const RingView& r, int n_q, int q_block0, int q_block_len,
                                   uint8_t* mask, hipStream_t s) {
  const size_t total = static_cast<size_t>(n_q) * r.N;
  const int blocks = static_cast<int>(std::min<size_t>((total + 255) / 256, 8192));
  hipLaunchKernelGGL(visibility_kernel, dim3(blocks), dim3(256), 0, s, r.slot_block, r.N, n_q, q_block0,
                     q_block_len, mask);
  return hipGetLastError();
}

}  // namespace rc
