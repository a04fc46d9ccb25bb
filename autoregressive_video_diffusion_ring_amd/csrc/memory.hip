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
//  * mass_prep_kernel: one wave per (head, 32 queries) rotates and quantises
//    the queries to FP8 (one scale per 32 queries) straight into the MFMA
//    operand order, with each query's -lse log2(e) and block id;
//  * key_mass_kernel: a workgroup of 16 waves owns 512 slots of one head
//    (32 per wave, K operand and factors in registers) and streams the
//    head's prepared queries through LDS, 8 tiles of 32 queries at a time,
//    double-buffered; per tile 2 MFMAs, then exp2(A s + b) summed in the lane.
// Each mass entry is summed by one lane pair in a fixed order (no atomics).
//
// Memory choice (memory_select_kernel, one workgroup) implements the greedy
// rule of the C ABI in closed form.  Within a block the greedy takes tokens
// in the order (score desc, slot asc); the k-th of them (rank k) has gain
// e = Q * gamma^k with gamma^k non-increasing in k, so along each block's
// list the key (e desc, rank asc, slot asc) increases, and taking the best
// block head each time is the same as taking the smallest keys overall.  So:
// sort the candidates by (block, score desc, slot) for the ranks, compute e,
// sort by (e desc, rank, slot) and keep the first min(M, C).  Scores are
// float64 sums over heads in head order and gamma^k the float64 product of k
// factors, as in the rule.  memory_move_kernel then copies the kept tokens of
// the ring part into the free memory slots.
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

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

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
};

template <int D>
__global__ __launch_bounds__(256) void mass_prep_kernel(MassArgs a) {
  using R = Rec<D>;
  const int lane = threadIdx.x % kWave;
  const int item = blockIdx.x * 4 + threadIdx.x / kWave;
  if (item >= a.H * a.QT) return;  // whole waves; no workgroup barrier below
  const int h = item / a.QT, t = item % a.QT;
  const int n = lane & 31, g = lane >> 5;
  const int qi = t * kMQ + n;
  const bool q_ok = qi < a.n_q;
  constexpr int NE = D / 2;  // values of this lane: d = 64 ks + 32 g + e, e < 32
  float x[NE];
  const uint16_t* qrow = a.q + (static_cast<size_t>(q_ok ? qi : 0) * a.H + h) * D;
  v4u raw[NE / 8];
#pragma unroll
  for (int r = 0; r < NE / 8; ++r)
    raw[r] = *reinterpret_cast<const v4u*>(qrow + (r / 4) * 64 + 32 * g + (r % 4) * 8);
  const long long qpos = static_cast<long long>(a.q_pos0) + qi;
#pragma unroll
  for (int e = 0; e < NE; e += 2) {
    const uint32_t w = raw[e / 8][(e / 2) % 4];
    const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
    float y0 = x0, y1 = x1;
    if (a.use_rope) {
      const int j = ((e / 32) * 64 + 32 * g + (e % 32)) >> 1;  // RoPE pair of (d, d + 1)
      float c, sn;
      rope_cs_hw(a.rope.rev[j], qpos, &c, &sn);
      y0 = x0 * c - x1 * sn;
      y1 = x0 * sn + x1 * c;
    }
    x[e] = q_ok ? y0 : 0.f;
    x[e + 1] = q_ok ? y1 : 0.f;
  }
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) am = fmaxf(am, fabsf(x[e]));
  am = group_max<kWave>(am);
  const float sq = am > 0.f ? am / 448.f : 1.f;
  const float iq = am > 0.f ? 448.f / am : 0.f;
  uint8_t* rec = a.ws + static_cast<size_t>(item) * R::bytes;
#pragma unroll
  for (int pc = 0; pc < NE / 16; ++pc) {
    v4u w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 16 * pc + 4 * k;
      w[k] = cvt_fp8x4(x[e] * iq, x[e + 1] * iq, x[e + 2] * iq, x[e + 3] * iq);
    }
    *reinterpret_cast<v4u*>(rec + R::frag + pc * 1024 + lane * 16) = w;
  }
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
__global__ __launch_bounds__(kMassThreads) void key_mass_kernel(MassArgs a) {
  using R = Rec<D>;
  constexpr int KS = D / 64;                               // MFMAs per tile
  constexpr int kBufBytes = kChunkTiles * R::bytes;
  constexpr int kLoads = (kBufBytes + kMassThreads * 16 - 1) / (kMassThreads * 16);
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 31, g = lane >> 5;
  int item = blockIdx.x;
  if (a.remap) item = (item % 8) * (a.items / 8) + item / 8;  // one head's groups on one XCD
  const int groups = a.v_ld / kMassSlots + (a.v_ld % kMassSlots != 0);
  const int h = item / groups;
  const int slot0 = (item % groups) * kMassSlots + 32 * wave;
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

  // prepared tiles of this head, in chunks of kChunkTiles through LDS
  const uint8_t* src = a.ws + static_cast<size_t>(h) * a.QT * R::bytes;
  const int n_chunks = (a.QT + kChunkTiles - 1) / kChunkTiles;
  auto chunk_bytes = [&](int c) { return min(kChunkTiles, a.QT - c * kChunkTiles) * R::bytes; };
  v4u stage[kLoads];
  auto fetch = [&](int c) {
    const int nb = chunk_bytes(c);
    const uint8_t* p = src + static_cast<size_t>(c) * kBufBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int off = (i * kMassThreads + tid) * 16;
      if (off < nb) stage[i] = *reinterpret_cast<const v4u*>(p + off);
    }
  };
  auto put = [&](uint8_t* dst, int c) {
    const int nb = chunk_bytes(c);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int off = (i * kMassThreads + tid) * 16;
      if (off < nb) *reinterpret_cast<v4u*>(dst + off) = stage[i];
    }
  };
  fetch(0);
  put(buf0, 0);
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

  for (int c = 0; c < n_chunks; ++c) {
    uint8_t* cur = (c & 1) ? buf1 : buf0;
    uint8_t* nxt = (c & 1) ? buf0 : buf1;
    const bool more = c + 1 < n_chunks;
    if (more) fetch(c + 1);
    const int tiles = min(kChunkTiles, a.QT - c * kChunkTiles);
    if (active)
      for (int t = 0; t < tiles; ++t) tile(cur + t * R::bytes);
    if (more) put(nxt, c + 1);
    __syncthreads();
  }
  // lanes n and n + 32 hold the same slot (different queries)
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
  const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (active && g == 0) {
    float* m = a.mass + static_cast<size_t>(h) * a.v_ld + slot;
    *m += total;
  }
}

// ------------------------------------------------------------ memory choice
constexpr int kSelThreads = 1024;
constexpr int kMaxCand = kMaxMemoryCandidates;

struct SelArgs {
  const int32_t* slot_block;
  const float* key_score;  // [H][v_ld]
  int H, v_ld;
  int A, E, N, M;  // anchor end, ring part end (first memory slot), slots, memory slots
  int head, n_new, rest;  // write range: head .. min(head + n, E) - 1, then A .. A + rest - 1
  float gamma;
  int32_t* moves;  // out: [0] = count, then (src, dst) pairs
};

// Exclusive prefix sum over the workgroup (every thread passes its value;
// returns the sum of the values of lower threads; `total` gets the sum).
__device__ int block_excl_scan(int v, int* sh, int* total) {
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
  for (int i = 0; i < kSelThreads / kWave; ++i) {
    const int t = sh[i];
    if (i < w) base += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}

__global__ __launch_bounds__(kSelThreads) void memory_select_kernel(SelArgs a) {
  __shared__ int32_t c_slot[kMaxCand];
  __shared__ int32_t c_blk[kMaxCand];
  __shared__ double c_val[kMaxCand];   // score Q, then e = Q gamma^rank
  __shared__ double g_pow[kMaxCand];   // gamma^r
  __shared__ int32_t c_rank[kMaxCand];
  __shared__ uint16_t order[kMaxCand];
  __shared__ int32_t flag[kMaxCand];   // per list position, reused
  __shared__ int sh[kSelThreads / kWave];
  __shared__ int s_count, s_maxrank;
  const int tid = threadIdx.x;
  constexpr int PER = kMaxCand / kSelThreads;  // list positions per thread

  // ---- candidates: occupied memory slots, then occupied slots of the write
  //      range, compacted in that order
  const int L = a.M + a.n_new;
  auto list_slot = [&](int j) {
    if (j < a.M) return a.E + j;
    const int i = j - a.M;
    return a.head + i < a.E ? a.head + i : a.A + (a.head + i - a.E);
  };
  int valid[PER], cnt = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = tid * PER + r;
    valid[r] = j < L && a.slot_block[list_slot(j)] != -1;
    cnt += valid[r];
  }
  int C;
  int pos = block_excl_scan(cnt, sh, &C);
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = tid * PER + r;
    if (valid[r]) {
      const int s = list_slot(j);
      c_slot[pos] = s;
      c_blk[pos] = a.slot_block[s];
      ++pos;
    }
  }
  __syncthreads();
  // ---- scores: float64 sums over heads, in head order
  for (int c = tid; c < C; c += kSelThreads) {
    const float* p = a.key_score + c_slot[c];
    double q = 0.0;
    for (int h = 0; h < a.H; ++h) q += static_cast<double>(p[static_cast<size_t>(h) * a.v_ld]);
    c_val[c] = q;
  }
  int P = 1;
  while (P < C) P <<= 1;
  for (int i = tid; i < P; i += kSelThreads) order[i] = static_cast<uint16_t>(i);
  if (tid == 0) s_maxrank = 0;
  __syncthreads();

  // bitonic sort of `order` (indices >= C sort last) by the comparator
  auto bitonic = [&](auto before) {
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kSelThreads) {
          const int l = i ^ j;
          if (l > i) {
            const int x = order[i], y = order[l];
            const bool up = (i & k) == 0;
            const bool y_first = y < C && (x >= C || before(y, x));
            const bool x_first = x < C && (y >= C || before(x, y));
            if (up ? y_first : x_first) {
              order[i] = static_cast<uint16_t>(y);
              order[l] = static_cast<uint16_t>(x);
            }
          }
        }
        __syncthreads();
      }
    }
  };
  // ---- ranks inside each block: order by (block, score desc, slot)
  bitonic([&](int x, int y) {
    if (c_blk[x] != c_blk[y]) return c_blk[x] < c_blk[y];
    if (c_val[x] != c_val[y]) return c_val[x] > c_val[y];
    return c_slot[x] < c_slot[y];
  });
  for (int p = tid; p < C; p += kSelThreads) {
    const int b = c_blk[order[p]];
    int lo = 0, hi = p;  // first position of block b
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (c_blk[order[mid]] < b) lo = mid + 1;
      else hi = mid;
    }
    c_rank[order[p]] = p - lo;
    atomicMax(&s_maxrank, p - lo);
  }
  __syncthreads();
  if (tid == 0) {  // gamma^r as the float64 product of r factors, in order
    const double gm = static_cast<double>(a.gamma);
    double gr = 1.0;
    for (int r = 0; r <= s_maxrank; ++r) {
      g_pow[r] = gr;
      gr *= gm;
    }
  }
  __syncthreads();
  for (int c = tid; c < C; c += kSelThreads) c_val[c] = c_val[c] * g_pow[c_rank[c]];
  for (int i = tid; i < P; i += kSelThreads) order[i] = static_cast<uint16_t>(i);
  __syncthreads();
  // ---- keep the first min(M, C) by (e desc, rank, slot)
  bitonic([&](int x, int y) {
    if (c_val[x] != c_val[y]) return c_val[x] > c_val[y];
    if (c_rank[x] != c_rank[y]) return c_rank[x] < c_rank[y];
    return c_slot[x] < c_slot[y];
  });
  const int K = min(a.M, C);
  // flag[j] for memory slot E + j: 1 = holds a kept token; for the write
  // range in ascending slot order (u < rest: A + u, then head + u - rest):
  // flag[M + u] = 1 = a kept token to move
  for (int j = tid; j < L; j += kSelThreads) flag[j] = 0;
  __syncthreads();
  for (int p = tid; p < K; p += kSelThreads) {
    const int s = c_slot[order[p]];
    if (s >= a.E) flag[s - a.E] = 1;
    else flag[a.M + (s >= a.head ? a.rest + (s - a.head) : s - a.A)] = 1;
  }
  __syncthreads();
  // free memory slots (no kept token) and incoming tokens, both ascending
  int f[PER], nf = 0, in[PER], ni = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = tid * PER + r;
    f[r] = j < a.M && flag[j] == 0;
    in[r] = j < a.n_new && flag[a.M + j] == 1;
    nf += f[r];
    ni += in[r];
  }
  int n_free, n_in;
  int fpos = block_excl_scan(nf, sh, &n_free);
  int ipos = block_excl_scan(ni, sh, &n_in);
  // the k-th incoming token goes to the k-th free slot; the free slots are
  // staged in c_slot (the candidate data is no longer needed)
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = tid * PER + r;
    if (f[r]) c_slot[fpos++] = a.E + j;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int u = tid * PER + r;
    if (in[r]) {
      const int s = u < a.rest ? a.A + u : a.head + (u - a.rest);
      a.moves[2 + 2 * ipos] = s;
      a.moves[3 + 2 * ipos] = c_slot[ipos];
      ++ipos;
    }
  }
  if (tid == 0) a.moves[0] = n_in;
}

// Copy kept tokens (K row, V^T column, scales, position, block) from the ring
// part to their memory slots: workgroup h handles head h.
template <int ES, int D>
__global__ __launch_bounds__(256) void memory_move_kernel(RingView r, const int32_t* moves) {
  const int h = blockIdx.x;
  const int count = moves[0];
  const int tid = threadIdx.x;
  uint8_t* k = static_cast<uint8_t*>(r.k) + static_cast<size_t>(h) * r.v_ld * D * ES;
  uint8_t* v = static_cast<uint8_t*>(r.v) + static_cast<size_t>(h) * D * r.v_ld * ES;
  constexpr int kPieces = D * ES / 16;  // 16-byte pieces per K row
  for (int i = tid; i < count * kPieces; i += 256) {
    const int m = i / kPieces, pc = i % kPieces;
    const int src = moves[2 + 2 * m], dst = moves[3 + 2 * m];
    *reinterpret_cast<v4u*>(k + static_cast<size_t>(dst) * D * ES + pc * 16) =
        *reinterpret_cast<const v4u*>(k + static_cast<size_t>(src) * D * ES + pc * 16);
  }
  for (int i = tid; i < count * D; i += 256) {
    const int m = i / D, j = i % D;
    const int src = moves[2 + 2 * m], dst = moves[3 + 2 * m];
    uint8_t* row = v + static_cast<size_t>(j) * r.v_ld * ES;
    if constexpr (ES == 1) row[dst] = row[src];
    else if constexpr (ES == 2) reinterpret_cast<uint16_t*>(row)[dst] = reinterpret_cast<const uint16_t*>(row)[src];
    else reinterpret_cast<uint32_t*>(row)[dst] = reinterpret_cast<const uint32_t*>(row)[src];
  }
  for (int m = tid; m < count; m += 256) {
    const int src = moves[2 + 2 * m], dst = moves[3 + 2 * m];
    if (r.k_scale) {
      r.k_scale[static_cast<size_t>(h) * r.v_ld + dst] = r.k_scale[static_cast<size_t>(h) * r.v_ld + src];
      r.v_scale[static_cast<size_t>(h) * r.v_ld + dst] = r.v_scale[static_cast<size_t>(h) * r.v_ld + src];
    }
    if (h == 0) {
      r.slot_pos[dst] = r.slot_pos[src];
      r.slot_block[dst] = r.slot_block[src];
    }
  }
}

template <int D>
hipError_t mass_impl(const RingView& r, const AttnCall& c, const float* lse, float* mass, hipStream_t s) {
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
  hipLaunchKernelGGL((mass_prep_kernel<D>), dim3((preps + 3) / 4), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups = (r.v_ld + kMassSlots - 1) / kMassSlots;
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

hipError_t launch_key_mass(const RingView& r, const AttnCall& c, const float* lse, float* mass, hipStream_t s) {
  if (r.kv == KV_FP8 && r.d == 128) return mass_impl<128>(r, c, lse, mass, s);
  if (r.kv == KV_FP8 && r.d == 64) return mass_impl<64>(r, c, lse, mass, s);
  return hipErrorInvalidValue;
}

size_t memory_workspace_bytes(int n_memory, int n_new) {
  if (n_memory <= 0) return 0;
  const size_t pairs = static_cast<size_t>(std::min(n_memory, n_new));
  return (8 + 8 * pairs + 255) / 256 * 256;
}

hipError_t launch_memory_update(const RingView& r, const float* key_score, float gamma, int head, int n_new,
                                void* workspace, hipStream_t s) {
  SelArgs a{};
  a.slot_block = r.slot_block;
  a.key_score = key_score;
  a.H = r.H;
  a.v_ld = r.v_ld;
  a.A = r.n_anchor;
  a.N = r.N;
  a.M = r.n_memory;
  a.E = r.N - r.n_memory;
  a.head = head;
  a.n_new = n_new;
  a.rest = std::max(0, head + n_new - a.E);
  a.gamma = gamma;
  a.moves = static_cast<int32_t*>(workspace);
  hipLaunchKernelGGL(memory_select_kernel, dim3(1), dim3(kSelThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t* mv = a.moves;
  switch (r.kv * 1000 + r.d) {
    case KV_FP8 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<1, 128>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    case KV_FP8 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<1, 64>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    case KV_BF16 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<2, 128>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    case KV_BF16 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<2, 64>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    case KV_F32 * 1000 + 128: hipLaunchKernelGGL((memory_move_kernel<4, 128>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    case KV_F32 * 1000 + 64: hipLaunchKernelGGL((memory_move_kernel<4, 64>), dim3(r.H), dim3(256), 0, s, r, mv); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rc
