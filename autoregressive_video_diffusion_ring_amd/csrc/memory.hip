// Scored content memory (gfx950): per-key attention mass, and the top-M
// choice of the tokens a layer keeps in its memory slots.
//
// StreamLTX project page, "Why a long take does not slow down": the long
// context is an anchor, a content memory and a FIFO of recent blocks; each
// layer scores its own keys on attention quality and temporal diversity and
// evicts down to a top-M budget.
//
// Attention mass.  mass[h][s] += sum_i p_h(i, s) with p normalised by the lse
// that the attention returned.  The attention kernel holds S^T (slots in
// accumulator rows, one query per lane), where a column sum over queries
// would cost a 32-lane reduction per slot and tile inside the hot loop; this
// separate kernel computes S = Q K^T instead, so that every lane holds ONE
// slot and 16 queries and the sum over queries stays in the lane:
//  * mass_prep_kernel: two waves per (head, 32 queries), one per half of the
//    head dimension, rotate and quantise the queries to FP8 (one scale per
//    32 queries, their absmax shared through LDS) straight into the MFMA
//    operand order, with each query's -lse log2(e) and block id;
//  * key_mass_kernel: a workgroup of 16 waves owns 512 slots of one head
//    (32 per wave, K operand and factors in registers) and streams the
//    head's prepared queries through LDS, 8 tiles of 32 queries at a time,
//    double-buffered with direct buffer-to-LDS loads (no staging registers,
//    so two workgroups fit on a compute unit: 8 waves per SIMD); per tile 2
//    MFMAs, then exp2(A s + b) summed in the lane.
// Each mass entry is summed by one lane pair in a fixed order (no atomics).
//
// Memory choice implements the greedy rule of the C ABI in closed form.
// Within a block the greedy takes tokens in the order (score desc, slot asc);
// the k-th of them (rank k) has gain e = Q * gamma^k with gamma^k
// non-increasing in k, so along each block's list the key (e desc, rank asc,
// slot asc) increases, and taking the best block head each time is the same
// as taking the smallest keys overall.  So a token's rank is the number of
// its block's tokens before it, its place in the final order the number of
// tokens with a smaller key, and it is kept when that place is below
// min(M, candidates): pairwise counts, spread over many workgroups
// (select_*_kernel), with no sort; gamma^rank is formed once per candidate.
// Scores are float64 sums over heads in head order and gamma^k the float32
// product of k factors, as in the rule.
// memory_move_kernel then copies the kept tokens of the ring part into the
// free memory slots.
#include <algorithm>
#include <cmath>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMinA = 0x1p-90f;  // floor of a slot's logit factor (zero keys)
constexpr int kMQ = 32;            // queries per prepared tile
constexpr int kMassWaves = 16;     // waves (x 32 slots) per mass workgroup
constexpr int kMassThreads = kMassWaves * kWave;
constexpr int kMassSlots = kMassWaves * 32;
constexpr int kChunkTiles = 8;     // prepared tiles per LDS buffer
constexpr int kMassListGroups = 64;  // slot groups a restricted call lists (else it runs all)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base` (raw; loads past the end
// return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from the buffer at lane offset off + uniform offset soff
// straight into LDS: the wave's 64 lanes fill the 1,024 bytes at lds_wave_base.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t soff, uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_wave_base), 16, static_cast<int>(off),
                                           static_cast<int>(soff), 0, 0);
}

// One prepared tile of 32 queries of one head:
//   [0, 16)    c_mul (float bits), block of the first and of the last query
//   [16, 144)  b[32]: -lse * log2(e) per query (-inf: padding or no key)
//   [144, 272) qb[32]: block id per query
//   [272, ..)  FP8 A operand: D/32 pieces of 64 lanes x 16 bytes; lane
//              (n, g) holds query n, d = 64 ks + 32 g + 16 part + 0..15 in
//              piece 2 ks + part
template <int D>
struct Rec {
  static constexpr int meta = 0, b = 16, qb = 144, frag = 272;
  static constexpr int bytes = frag + (D / 32) * 1024;
};

struct MassArgs {
  const uint8_t* k;           // [H][v_ld][D] codes
  const float* k_scale;       // [H][v_ld]
  const int32_t* slot_block;  // [v_ld]
  const uint16_t* q;          // [n_q][H][D] bf16
  const float* lse;           // [H][n_q]
  float* mass;                // [H][v_ld]
  uint8_t* ws;                // [H][QT] prepared tiles
  int H, v_ld, n_q, QT, q_pos0, q_block0, q_block_len;
  int items, remap;
  float bias_log2, scale_log2;
  int use_rope;
  RopeTable rope;
  // optional restriction to slot ranges [lo, hi): only the slot groups that
  // meet a range run (n_groups of them, listed), and only slots inside a
  // range receive mass
  int n_ranges, range_lo[kMassRanges], range_hi[kMassRanges];
  int n_groups;
  int16_t group_id[kMassListGroups];
};

template <int D>
__global__ __launch_bounds__(256) void mass_prep_kernel(MassArgs a) {
  // two waves per prepared tile: wave half w rotates and quantises the head
  // dimension's half d = 64 w .. 64 w + 63 (the pieces 2 w, 2 w + 1 of the
  // operand); the tile's absmax is shared through LDS
  using R = Rec<D>;
  constexpr int KS = D / 64;
  static_assert(KS <= 2, "one or two halves of the head dimension");
  __shared__ float amax_sh[2][2];
  const int lane = threadIdx.x % kWave;
  const int local = threadIdx.x / (2 * kWave);      // tile of this workgroup (0, 1)
  const int w = (threadIdx.x / kWave) % 2;          // half of the head dimension
  const int item = blockIdx.x * 2 + local;
  const bool item_ok = item < a.H * a.QT;            // the workgroup's barrier is reached by every wave
  const int it = item_ok ? item : 0;
  const int h = it / a.QT, t = it % a.QT;
  const int n = lane & 31, g = lane >> 5;
  const int qi = t * kMQ + n;
  const bool q_ok = item_ok && qi < a.n_q;
  const bool live = w < KS;                         // d 64: one half only
  constexpr int NE = 32;  // values of this lane: d = 64 w + 32 g + e, e < 32
  float x[NE];
  const uint16_t* qrow = a.q + (static_cast<size_t>(q_ok ? qi : 0) * a.H + h) * D;
  v4u raw[NE / 8];
#pragma unroll
  for (int r = 0; r < NE / 8; ++r)
    raw[r] = live ? *reinterpret_cast<const v4u*>(qrow + 64 * w + 32 * g + r * 8) : v4u{0u, 0u, 0u, 0u};
  const long long qpos = static_cast<long long>(a.q_pos0) + qi;
#pragma unroll
  for (int e = 0; e < NE; e += 2) {
    const uint32_t wd = raw[e / 8][(e / 2) % 4];
    const float x0 = __uint_as_float(wd << 16), x1 = __uint_as_float(wd & 0xFFFF0000u);
    float y0 = x0, y1 = x1;
    if (a.use_rope) {
      const int j = (64 * w + 32 * g + e) >> 1;  // RoPE pair of (d, d + 1)
      float c, sn;
      rope_cs_hw(a.rope.rev[live ? j : 0], qpos, &c, &sn);
      y0 = x0 * c - x1 * sn;
      y1 = x0 * sn + x1 * c;
    }
    x[e] = q_ok && live ? y0 : 0.f;
    x[e + 1] = q_ok && live ? y1 : 0.f;
  }
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) am = fmaxf(am, fabsf(x[e]));
  am = group_max<kWave>(am);
  if (lane == 0) amax_sh[local][w] = am;
  __syncthreads();
  am = fmaxf(amax_sh[local][0], amax_sh[local][1]);
  if (!item_ok || !live) return;
  const float sq = am > 0.f ? am / 448.f : 1.f;
  const float iq = am > 0.f ? 448.f / am : 0.f;
  uint8_t* rec = a.ws + static_cast<size_t>(item) * R::bytes;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    v4u wv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 16 * part + 4 * k;
      wv[k] = cvt_fp8x4(x[e] * iq, x[e + 1] * iq, x[e + 2] * iq, x[e + 3] * iq);
    }
    *reinterpret_cast<v4u*>(rec + R::frag + (2 * w + part) * 1024 + lane * 16) = wv;
  }
  if (w != 0) return;
  const int last = min(t * kMQ + kMQ, a.n_q) - 1;
  const int qb_lo = a.q_block0 + (t * kMQ) / a.q_block_len;
  const int qb_hi = a.q_block0 + last / a.q_block_len;
  if (lane == 0)
    *reinterpret_cast<v4i*>(rec + R::meta) = v4i{__float_as_int(a.scale_log2 * sq), qb_lo, qb_hi, 0};
  if (g == 0) {
    const float l = q_ok ? a.lse[static_cast<size_t>(h) * a.n_q + qi] : -INFINITY;
    reinterpret_cast<float*>(rec + R::b)[n] = l == -INFINITY ? -INFINITY : -l * kLog2e;
    reinterpret_cast<int32_t*>(rec + R::qb)[n] = a.q_block0 + (q_ok ? qi : last) / a.q_block_len;
  }
}

template <int D>
__global__ __launch_bounds__(kMassThreads, 8) void key_mass_kernel(MassArgs a) {
  using R = Rec<D>;
  constexpr int KS = D / 64;                               // MFMAs per tile
  constexpr int kChunkBytes = kChunkTiles * R::bytes;      // prepared bytes per chunk
  constexpr int kBufBytes = (kChunkBytes + 1023) / 1024 * 1024;  // whole 1 KiB wave loads
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 31, g = lane >> 5;
  int item = blockIdx.x;
  if (a.remap) item = (item % 8) * (a.items / 8) + item / 8;  // one head's groups on one XCD
  const int groups = a.n_groups > 0 ? a.n_groups : a.v_ld / kMassSlots + (a.v_ld % kMassSlots != 0);
  const int h = item / groups;
  const int grp = a.n_groups > 0 ? a.group_id[item % groups] : item % groups;
  const int slot0 = grp * kMassSlots + 32 * wave;
  const bool active = slot0 < a.v_ld;  // v_ld is a multiple of 64: a wave's slots are all real or all absent
  const int slot = active ? slot0 + n : 0;

  // this lane's slot: K operand (d = 64 ks + 32 g .. +31), scale, block
  v8i kf[KS];
  const uint8_t* krow = a.k + (static_cast<size_t>(h) * a.v_ld + slot) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const v4i lo = *reinterpret_cast<const v4i*>(krow + 64 * ks + 32 * g);
    const v4i hi = *reinterpret_cast<const v4i*>(krow + 64 * ks + 32 * g + 16);
    kf[ks] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  const float ksc = a.k_scale[static_cast<size_t>(h) * a.v_ld + slot];
  const int kb = a.slot_block[slot];

  // prepared tiles of this head, in chunks of kChunkTiles through LDS: the
  // chunk's bytes in 1 KiB pieces, piece p loaded by wave p % 16 (a piece
  // that runs past the head's tiles reads zeros; bytes past the chunk land
  // in the buffer's unused tail or belong to tiles the loop does not visit)
  const uint8_t* src = a.ws + static_cast<size_t>(h) * a.QT * R::bytes;
  const __amdgpu_buffer_rsrc_t src_rsrc = make_rsrc(src, static_cast<uint32_t>(a.QT) * R::bytes);
  const int n_chunks = (a.QT + kChunkTiles - 1) / kChunkTiles;
  auto chunk_bytes = [&](int c) { return min(kChunkTiles, a.QT - c * kChunkTiles) * R::bytes; };
  auto issue = [&](uint8_t* dst, int c) __attribute__((always_inline)) {
    const int nb = chunk_bytes(c);
    for (int p = wave; p * 1024 < nb; p += kMassWaves)
      dma16(src_rsrc, static_cast<uint32_t>(lane * 16), static_cast<uint32_t>(c * kChunkBytes + p * 1024),
            dst + p * 1024);
  };
  issue(buf0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's pieces are in LDS
  __syncthreads();

  float acc = 0.f;
  auto tile = [&](const uint8_t* rec) {
    const v4i meta = *reinterpret_cast<const v4i*>(rec + R::meta);
    const float c_mul = __int_as_float(__builtin_amdgcn_readfirstlane(meta.x));
    const int qb_lo = __builtin_amdgcn_readfirstlane(meta.y);
    const int qb_hi = __builtin_amdgcn_readfirstlane(meta.z);
    const float A = fmaxf(c_mul * ksc, kMinA);
    const bool uniform = qb_lo == qb_hi;
    // uniform block: the bias enters the accumulator's start value (A C = bias)
    const bool vis_u = kb != -1 && kb <= qb_lo;
    const float cinit = uniform && kb < qb_lo ? a.bias_log2 * __builtin_amdgcn_rcpf(A) : 0.f;
    v16f s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = cinit;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const v4i lo = *reinterpret_cast<const v4i*>(rec + R::frag + (2 * ks) * 1024 + lane * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(rec + R::frag + (2 * ks + 1) * 1024 + lane * 16);
      const v8i qa = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kf[ks], s, 0, 0, 0, 0, 0, 0);
    }
    // accumulator element e of lane (n, g) is query 8 (e / 4) + 4 g + e % 4, slot n
    const float* bq = reinterpret_cast<const float*>(rec + R::b);
    float sum = 0.f;
    if (uniform) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f b = *reinterpret_cast<const v4f*>(bq + 8 * j + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(fmaf(s[4 * j + i], A, b[i]));
      }
      acc += vis_u ? sum : 0.f;
    } else {
      const int32_t* qbs = reinterpret_cast<const int32_t*>(rec + R::qb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f b = *reinterpret_cast<const v4f*>(bq + 8 * j + 4 * g);
        const v4i qb = *reinterpret_cast<const v4i*>(qbs + 8 * j + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float z = fmaf(s[4 * j + i], A, b[i]);
          z = kb < qb[i] ? z + a.bias_log2 : z;
          const bool vis = kb != -1 && kb <= qb[i];
          sum += vis ? __builtin_amdgcn_exp2f(z) : 0.f;
        }
      }
      acc += sum;
    }
  };

  // one chunk from cur while the next one loads into nxt; the two buffers
  // alternate by call site, so that each LDS read waits only for the loads
  // into its own buffer
  auto chunk = [&](const uint8_t* cur, uint8_t* nxt, int c) __attribute__((always_inline)) {
    if (c + 1 < n_chunks) issue(nxt, c + 1);
    const int tiles = min(kChunkTiles, a.QT - c * kChunkTiles);
    if (active)
      for (int t = 0; t < tiles; ++t) tile(cur + t * R::bytes);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // chunk c + 1 is in nxt; every wave is done with cur
  };
  for (int c = 0; c < n_chunks; c += 2) {
    chunk(buf0, buf1, c);
    if (c + 1 < n_chunks) chunk(buf1, buf0, c + 1);
  }
  // lanes n and n + 32 hold the same slot (different queries)
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
  const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  bool wanted = a.n_ranges == 0;
#pragma unroll
  for (int i = 0; i < kMassRanges; ++i)
    wanted = wanted || (i < a.n_ranges && slot >= a.range_lo[i] && slot < a.range_hi[i]);
  if (active && g == 0 && wanted) {
    float* m = a.mass + static_cast<size_t>(h) * a.v_ld + slot;
    *m += total;
  }
}

// ------------------------------------------------------------ memory choice
// The list positions c < L = M + n: c < M is memory slot E + c, M + i the
// i-th slot of the write (head + i, wrapping from E to A); a position is a
// candidate when its slot holds a token.  Every decision is an integer count
// over pairs of candidates, added with integer atomics (exact, so the result
// does not depend on the order in which workgroups run):
//   rank[c] = candidates of c's block before c in (score desc, slot asc),
//   pos[c]  = candidates before c in (e desc, rank asc, slot asc),
//             e = score * gamma^rank;
// c is kept when pos[c] < K = min(M, candidates).
constexpr int kSelBlock = 256;  // candidates per workgroup, one per thread
constexpr int kSelChunk = 64;   // candidates each wave compares against (one per lane)
constexpr int kMoveRows = 8;    // V^T rows per move workgroup

struct SelArgs {
  const int32_t* slot_block;
  const float* key_score;  // [H][v_ld]
  int H, v_ld;
  int A, E, M;             // anchor end, ring part end (first memory slot), memory slots
  int head, n_new, rest;   // the write: head .. min(head + n, E) - 1, then A .. A + rest - 1
  int L, K;                // M + n; tokens kept, min(M, candidates)
  float gamma;
  double* score;           // workspace arrays of L entries
  double* gain;            // e = score * gamma^rank
  int32_t* slot;
  int32_t* blk;            // -1: not a candidate
  int32_t* rank;
  int32_t* pos;
};

__device__ __forceinline__ int list_slot(const SelArgs& a, int c) {
  if (c < a.M) return a.E + c;
  const int i = c - a.M;
  return a.head + i < a.E ? a.head + i : a.A + (a.head + i - a.E);
}

// gamma^r as the float32 product of r factors, left to right (a dependent
// chain of float32 multiplies: far shorter in latency than float64)
__device__ __forceinline__ float gamma_pow(float g, int r) {
  if (g == 1.f) return 1.f;
  float x = 1.f;
  int i = 0;
  for (; i + 16 <= r; i += 16) {  // unrolled: one branch per 16 dependent multiplies
#pragma unroll
    for (int u = 0; u < 16; ++u) x *= g;
  }
  for (; i < r; ++i) x *= g;
  return x;
}

// Candidates and their scores (float64 sums over heads, in head order).
__global__ __launch_bounds__(kSelBlock) void select_score_kernel(SelArgs a) {
  const int c = blockIdx.x * kSelBlock + threadIdx.x;
  if (c >= a.L) return;
  const int s = list_slot(a, c);
  const int b = a.slot_block[s];
  double q = 0.0;
  if (b != -1) {
    const float* p = a.key_score + s;
    int h = 0;
    for (; h + 8 <= a.H; h += 8) {  // eight loads in flight, then the sums in order
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = p[static_cast<size_t>(h + k) * a.v_ld];
#pragma unroll
      for (int k = 0; k < 8; ++k) q += static_cast<double>(v[k]);
    }
    for (; h < a.H; ++h) q += static_cast<double>(p[static_cast<size_t>(h) * a.v_ld]);
  }
  a.score[c] = q;
  a.slot[c] = s;
  a.blk[c] = b;
  a.rank[c] = 0;
  a.pos[c] = 0;
}

// The chunk's candidates are held one per lane and broadcast with readlane
// (scalar registers), so the inner loop reads no memory.
__device__ __forceinline__ int rl(int x, int k) { return __builtin_amdgcn_readlane(x, k); }
__device__ __forceinline__ double rld(double x, int k) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = rl(static_cast<int>(u & 0xFFFFFFFFu), k), hi = rl(static_cast<int>(u >> 32), k);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// rank[c] += candidates of the chunk in c's block that come before c.
__global__ __launch_bounds__(kSelBlock) void select_rank_kernel(SelArgs a) {
  const int lane = threadIdx.x % kWave;
  const int o = blockIdx.y * kSelChunk + lane;
  const bool o_in = o < a.L;
  const double oq = o_in ? a.score[o] : 0.0;
  const int os = o_in ? a.slot[o] : 0, ob = o_in ? a.blk[o] : -1;
  const int c = blockIdx.x * kSelBlock + threadIdx.x;
  const bool in = c < a.L;
  const int b = in ? a.blk[c] : -1;
  const double q = in ? a.score[c] : 0.0;
  const int s = in ? a.slot[c] : 0;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kSelChunk; ++k) {
    const int kb = rl(ob, k);
    const double kq = rld(oq, k);
    const int ks = rl(os, k);
    cnt += kb == b && (kq > q || (kq == q && ks < s));
  }
  if (b != -1 && cnt) atomicAdd(&a.rank[c], cnt);
}

// e = score * gamma^rank, once per candidate.
__global__ __launch_bounds__(kSelBlock) void select_gain_kernel(SelArgs a) {
  const int c = blockIdx.x * kSelBlock + threadIdx.x;
  if (c >= a.L) return;
  a.gain[c] = a.blk[c] != -1 ? a.score[c] * static_cast<double>(gamma_pow(a.gamma, a.rank[c])) : 0.0;
}

// pos[c] += candidates of the chunk that come before c in the final order.
__global__ __launch_bounds__(kSelBlock) void select_pos_kernel(SelArgs a) {
  const int lane = threadIdx.x % kWave;
  const int o = blockIdx.y * kSelChunk + lane;
  const bool o_in = o < a.L && a.blk[o] != -1;
  const double oe = o_in ? a.gain[o] : 0.0;
  const int orank = o_in ? a.rank[o] : 0, os = o_in ? a.slot[o] : 0, ov = o_in;
  const int c = blockIdx.x * kSelBlock + threadIdx.x;
  const bool in = c < a.L && a.blk[c] != -1;
  const double e = in ? a.gain[c] : 0.0;
  const int r = in ? a.rank[c] : 0, s = in ? a.slot[c] : 0;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kSelChunk; ++k) {
    const double ke = rld(oe, k);
    const int kr = rl(orank, k), ks = rl(os, k), kv = rl(ov, k);
    cnt += kv && (ke > e || (ke == e && (kr < r || (kr == r && ks < s))));
  }
  if (in && cnt) atomicAdd(&a.pos[c], cnt);
}

// Exclusive prefix sum over a 256-thread workgroup; `total` gets the sum.
__device__ int wg_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) sh[w] = x;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = sh[i];
    if (i < w) base += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}

// Workgroup (h, group): every workgroup pairs the k-th kept token of the
// ring part (ascending slot) with the k-th memory slot that holds no kept
// token (ascending), then copies its share for head h: V^T rows
// group*8 .. +7, a share of the K rows, and (group 0) the scales and (head 0)
// positions and blocks.
template <int ES, int D>
__global__ __launch_bounds__(256) void memory_move_kernel(RingView r, SelArgs a) {
  __shared__ int32_t src_s[kMaxMemoryCandidates];
  __shared__ int32_t dst_s[kMaxMemoryCandidates];
  __shared__ int sh[4];
  constexpr int G = D / kMoveRows;
  const int h = blockIdx.x / G, grp = blockIdx.x % G;
  const int tid = threadIdx.x;
  auto kept = [&](int c) { return a.blk[c] != -1 && a.pos[c] < a.K; };
  int n_free = 0, n_in = 0;
  for (int base = 0; base < a.M; base += 256) {
    const int j = base + tid;
    const int f = j < a.M && !kept(j);
    int tot;
    const int at = wg_excl_scan(f, sh, &tot);
    if (f) dst_s[n_free + at] = a.E + j;
    n_free += tot;
  }
  for (int base = 0; base < a.n_new; base += 256) {
    const int u = base + tid;  // ascending slots: the wrapped part A.., then head..
    int f = 0, s = 0;
    if (u < a.n_new) {
      const int i = u < a.rest ? (a.E - a.head) + u : u - a.rest;
      s = u < a.rest ? a.A + u : a.head + (u - a.rest);
      f = kept(a.M + i);
    }
    int tot;
    const int at = wg_excl_scan(f, sh, &tot);
    if (f) src_s[n_in + at] = s;
    n_in += tot;
  }
  __syncthreads();
  const int pairs = min(n_in, n_free);
  uint8_t* k = static_cast<uint8_t*>(r.k) + static_cast<size_t>(h) * r.v_ld * D * ES;
  uint8_t* v = static_cast<uint8_t*>(r.v) + static_cast<size_t>(h) * D * r.v_ld * ES;
  // V^T: rows grp*8 .. +7 of every pair, loads first
  for (int m = tid; m < pairs; m += 256) {
    const int src = src_s[m], dst = dst_s[m];
    uint32_t x[kMoveRows];
#pragma unroll
    for (int j = 0; j < kMoveRows; ++j) {
      const uint8_t* row = v + static_cast<size_t>(grp * kMoveRows + j) * r.v_ld * ES;
      if constexpr (ES == 1) x[j] = row[src];
      else if constexpr (ES == 2) x[j] = reinterpret_cast<const uint16_t*>(row)[src];
      else x[j] = reinterpret_cast<const uint32_t*>(row)[src];
    }
#pragma unroll
    for (int j = 0; j < kMoveRows; ++j) {
      uint8_t* row = v + static_cast<size_t>(grp * kMoveRows + j) * r.v_ld * ES;
      if constexpr (ES == 1) row[dst] = static_cast<uint8_t>(x[j]);
      else if constexpr (ES == 2) reinterpret_cast<uint16_t*>(row)[dst] = static_cast<uint16_t>(x[j]);
      else reinterpret_cast<uint32_t*>(row)[dst] = x[j];
    }
  }
  // K rows: 16-byte pieces, spread over the G workgroups of the head
  constexpr int KP = D * ES / 16;
  for (int i0 = grp * 256 + tid; i0 < pairs * KP; i0 += 4 * G * 256) {
    v4u x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * G * 256;
      if (i < pairs * KP)
        x[u] = *reinterpret_cast<const v4u*>(k + static_cast<size_t>(src_s[i / KP]) * D * ES + (i % KP) * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * G * 256;
      if (i < pairs * KP)
        *reinterpret_cast<v4u*>(k + static_cast<size_t>(dst_s[i / KP]) * D * ES + (i % KP) * 16) = x[u];
    }
  }
  if (grp == 0) {
    for (int m = tid; m < pairs; m += 256) {
      const int src = src_s[m], dst = dst_s[m];
      if (r.k_scale) {
        const size_t o = static_cast<size_t>(h) * r.v_ld;
        const float ks = r.k_scale[o + src], vs = r.v_scale[o + src];
        r.k_scale[o + dst] = ks;
        r.v_scale[o + dst] = vs;
      }
      if (h == 0) {
        const int p = r.slot_pos[src], b = r.slot_block[src];
        r.slot_pos[dst] = p;
        r.slot_block[dst] = b;
      }
    }
  }
}

template <int D>
hipError_t mass_impl(const RingView& r, const AttnCall& c, const float* lse, float* mass, const int* ranges,
                     int n_ranges, hipStream_t s) {
  MassArgs a{};
  a.k = static_cast<const uint8_t*>(r.k);
  a.k_scale = r.k_scale;
  a.slot_block = r.slot_block;
  a.q = static_cast<const uint16_t*>(c.q);
  a.lse = lse;
  a.mass = mass;
  a.ws = static_cast<uint8_t*>(c.workspace);
  a.H = r.H;
  a.v_ld = r.v_ld;
  a.n_q = c.n_q;
  a.QT = (c.n_q + kMQ - 1) / kMQ;
  a.q_pos0 = c.q_pos0;
  a.q_block0 = c.q_block0;
  a.q_block_len = c.q_block_len;
  const float sigma = c.softmax_scale != 0.f ? c.softmax_scale : 1.f / std::sqrt(static_cast<float>(D));
  a.scale_log2 = sigma * kLog2e;
  a.bias_log2 = c.cache_bias * kLog2e;
  a.use_rope = r.rope_base > 0.f;
  for (int j = 0; j < D / 2; ++j)
    a.rope.rev[j] = a.use_rope ? std::pow(static_cast<double>(r.rope_base), -2.0 * j / D) / (2.0 * M_PI) : 0.0;
  const int preps = r.H * a.QT;
  hipLaunchKernelGGL((mass_prep_kernel<D>), dim3((preps + 1) / 2), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int groups = (r.v_ld + kMassSlots - 1) / kMassSlots;
  a.n_ranges = n_ranges;
  if (n_ranges > 0) {
    for (int i = 0; i < n_ranges; ++i) {
      a.range_lo[i] = ranges[2 * i];
      a.range_hi[i] = ranges[2 * i + 1];
    }
    int listed = 0;
    for (int gi = 0; gi < groups; ++gi) {
      bool meets = false;
      for (int i = 0; i < n_ranges; ++i)
        meets = meets || (a.range_lo[i] < (gi + 1) * kMassSlots && a.range_hi[i] > gi * kMassSlots);
      if (meets && listed < kMassListGroups) a.group_id[listed] = static_cast<int16_t>(gi);
      listed += meets ? 1 : 0;
    }
    if (listed == 0) return hipSuccess;  // nothing to compute
    if (listed <= kMassListGroups) {
      a.n_groups = listed;
      groups = listed;
    }  // else: every group runs; the range test still limits what is written
  }
  a.items = r.H * groups;
  a.remap = a.items % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL((key_mass_kernel<D>), dim3(a.items), dim3(kMassThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool key_mass_supported(int kv, int d) { return kv == KV_FP8 && (d == 64 || d == 128); }

size_t key_mass_workspace_bytes(const RingView& r, int n_q) {
  if (!key_mass_supported(r.kv, r.d) || n_q < 1) return 0;
  const size_t rec = r.d == 128 ? Rec<128>::bytes : Rec<64>::bytes;
  return static_cast<size_t>(r.H) * ((n_q + kMQ - 1) / kMQ) * rec;
}

hipError_t launch_key_mass(const RingView& r, const AttnCall& c, const float* lse, float* mass, const int* ranges,
                           int n_ranges, hipStream_t s) {
  if (r.kv == KV_FP8 && r.d == 128) return mass_impl<128>(r, c, lse, mass, ranges, n_ranges, s);
  if (r.kv == KV_FP8 && r.d == 64) return mass_impl<64>(r, c, lse, mass, ranges, n_ranges, s);
  return hipErrorInvalidValue;
}

size_t memory_workspace_bytes(int n_memory, int n_new) {
  if (n_memory <= 0) return 0;
  const size_t L = static_cast<size_t>(n_memory) + n_new;
  return (L * (2 * 8 + 4 * 4) + 255) / 256 * 256;
}

hipError_t launch_memory_update(const RingView& r, const float* key_score, float gamma, int head, int n_new,
                                int n_candidates, void* workspace, hipStream_t s) {
  SelArgs a{};
  a.slot_block = r.slot_block;
  a.key_score = key_score;
  a.H = r.H;
  a.v_ld = r.v_ld;
  a.A = r.n_anchor;
  a.M = r.n_memory;
  a.E = r.N - r.n_memory;
  a.head = head;
  a.n_new = n_new;
  a.rest = std::max(0, head + n_new - a.E);
  a.L = a.M + n_new;
  a.K = std::min(a.M, n_candidates);
  a.gamma = gamma;
  a.score = static_cast<double*>(workspace);
  a.gain = a.score + a.L;
  a.slot = reinterpret_cast<int32_t*>(a.gain + a.L);
  a.blk = a.slot + a.L;
  a.rank = a.blk + a.L;
  a.pos = a.rank + a.L;
  const int nb = (a.L + kSelBlock - 1) / kSelBlock, nc = (a.L + kSelChunk - 1) / kSelChunk;
  hipLaunchKernelGGL(select_score_kernel, dim3(nb), dim3(kSelBlock), 0, s, a);
  hipLaunchKernelGGL(select_rank_kernel, dim3(nb, nc), dim3(kSelBlock), 0, s, a);
  hipLaunchKernelGGL(select_gain_kernel, dim3(nb), dim3(kSelBlock), 0, s, a);
  hipLaunchKernelGGL(select_pos_kernel, dim3(nb, nc), dim3(kSelBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(r.H * (r.d / kMoveRows));
  switch (r.kv * 1000 + r.d) {
    case KV_FP8 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<1, 128>), grid, dim3(256), 0, s, r, a); break;
    case KV_FP8 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<1, 64>), grid, dim3(256), 0, s, r, a); break;
    case KV_BF16 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<2, 128>), grid, dim3(256), 0, s, r, a); break;
    case KV_BF16 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<2, 64>), grid, dim3(256), 0, s, r, a); break;
    case KV_F32 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<4, 128>), grid, dim3(256), 0, s, r, a); break;
    case KV_F32 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<4, 64>), grid, dim3(256), 0, s, r, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rc
