// Ring-cache write, delta re-rotation and clear kernels (gfx950).
//
// The write moves each chunk's new K and V into the ring once, applying RoPE
// to K and FP8 quantisation to both at write time, and the re-rotation moves
// every cached key to new positions by a delta rotation (Runway Characters,
// abstract).  Both are HBM-bound: each byte of input is read once and each
// byte of the cache written once, so both are organised to keep many loads
// in flight: every thread issues all of its loads before any arithmetic.
//
// Write layout: the written range is cut into at most two linear slot
// ranges, [head, min(head + n, E)) and the part past slot E-1 (E = N, or the
// first content-memory slot), which wraps to the first slot of the ring part
// (slot 0, or the first slot after the pinned anchor slots), and each range
// into 32-slot chunks aligned to multiples of 32.  One workgroup handles one chunk for kWHeads heads:
//  * a row (one token of one head, d elements) is handled by 16 lanes with
//    d/16 contiguous elements each, so a row's loads and stores are whole
//    contiguous cache rows; a thread takes 4 consecutive slots of one head;
//  * each RoPE angle is reduced in float64 to at most half a revolution and
//    finished by the hardware sine and cosine (which take revolutions; their
//    error on that range is about 2^-23, the same as float32 rounding of the
//    angle itself);
//  * V is quantised the same way, transposed through LDS (a thread writes the
//    4 slots of one d as one word) and stored to the [H][d][v_ld] layout as
//    16-byte pieces (chunks start on a multiple of 32 and v_ld is a multiple
//    of 64, so pieces are aligned).
#include <algorithm>
#include <cmath>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

constexpr int kThreads = 256;
constexpr int kWChunk = 32;                  // slots per write workgroup
constexpr int kWHeads = 2;                   // heads per write workgroup
constexpr int kLanesPerRow = 16;
constexpr int kRowGroups = kThreads / kLanesPerRow;
constexpr int kRowsPerThread = kWChunk * kWHeads / kRowGroups;  // consecutive slots
constexpr int kSlotGroups = kWChunk / kRowsPerThread;  // row groups per head
static_assert(kRowsPerThread == 4 && kSlotGroups * kWHeads == kRowGroups, "thread -> rows");

template <int KV>
struct Store;
template <>
struct Store<KV_F32> {
  static constexpr int bytes = 4;
};
template <>
struct Store<KV_BF16> {
  static constexpr int bytes = 2;
};
template <>
struct Store<KV_FP8> {
  static constexpr int bytes = 1;
};

struct WriteArgs {
  RingView r;
  const void* k_new;
  const void* v_new;
  int n_new, head, pos0, block_id;
  int lo_a, hi_a, lo_b, hi_b, chunks_a;
  int wrap_tok;       // token index of slot lo_b minus lo_b + head (the wrapped range's offset)
  int chunks, items;  // chunks per head group; chunks x head groups
  int grid;           // workgroups launched (a multiple of 8)
  int use_rope;
  RopeTable rope;
};

// Raw input words of one row piece: EPL elements, bf16 pairs or floats.
template <int KV, int EPL>
struct Raw {
  static constexpr int words = KV == KV_F32 ? EPL : EPL / 2;
  uint32_t w[words];
};

template <int KV, int EPL>
__device__ __forceinline__ void load_raw(const void* base, size_t elem_off, Raw<KV, EPL>& r) {
  constexpr int W = Raw<KV, EPL>::words;
  const uint8_t* p = static_cast<const uint8_t*>(base) + elem_off * (KV == KV_F32 ? 4 : 2);
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 t = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i] = t.x;
      r.w[4 * i + 1] = t.y;
      r.w[4 * i + 2] = t.z;
      r.w[4 * i + 3] = t.w;
    }
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    r.w[0] = t.x;
    r.w[1] = t.y;
  }
}

template <int KV, int EPL>
__device__ __forceinline__ void unpack(const Raw<KV, EPL>& r, float* x) {
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = __uint_as_float(r.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
      x[2 * i] = __uint_as_float(r.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
    }
  }
}

// Encodes EPL values as FP8 codes of the given scale.  EXACT: correctly
// rounded codes of the exact quotients (needed where inputs are short
// binary fractions, so that ties are common); otherwise the float32 product
// x * (1/scale), within a few float32 ulps of the quotient, is converted
// directly (used for keys that were just rotated in float32, whose values
// already carry float32 rounding and essentially never sit on a tie).
template <int EPL, bool EXACT>
__device__ __forceinline__ void encode_fp8(const float* x, float sc, float rcp, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) {
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = EXACT ? qdiv_rto(x[4 * i + k], sc, rcp) : x[4 * i + k] * rcp;
    w[i] = cvt_fp8x4(q[0], q[1], q[2], q[3]);
  }
}

// Stores EPL values of a K row piece: FP8 codes, bf16 or float32.
template <int KV, int EPL, bool EXACT>
__device__ __forceinline__ void store_row(void* base, size_t elem_off, const float* x, float sc, float rcp) {
  if constexpr (KV == KV_FP8) {
    uint32_t w[EPL / 4];
    encode_fp8<EPL, EXACT>(x, sc, rcp, w);
    uint8_t* p = static_cast<uint8_t*>(base) + elem_off;
    if constexpr (EPL == 16) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    else if constexpr (EPL == 8) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint32_t*>(p) = w[0];
  } else if constexpr (KV == KV_BF16) {
    uint16_t* p = static_cast<uint16_t*>(base) + elem_off;
    if constexpr (EPL == 8) {
      *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
    } else {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    }
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) p[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  }
}

// Absmax over the LANES lanes of a row -> scale = max|x| / 448 in float32
// (IEEE division); a zero row gives 0.
template <int LANES, int EPL>
__device__ __forceinline__ float row_scale(const float* x) {
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
  if constexpr (LANES == 4 || LANES == 8 || LANES == 16) a = group_max_dpp<LANES>(a);  // rows are aligned lane groups
  else a = group_max<LANES>(a);
  return div448(a);
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(WriteArgs a) {
  constexpr int EPL = D / kLanesPerRow;
  constexpr int ES = Store<KV>::bytes;
  // V^T rows of the chunk: row (head, j) holds the chunk's slots, padded by
  // 4 slots against bank conflicts of the transposing writes
  constexpr int RS = (kWChunk + 4) * ES;
  __shared__ __attribute__((aligned(16))) uint8_t vt[kWHeads * D * RS];

  const int tid = threadIdx.x;
  // Every argument used before the first input load is read here in one
  // batch of scalar loads; the empty asm keeps them from being spread over
  // the dependent steps below (one argument round trip instead of several).
  const int H = a.r.H, grid = a.grid, items = a.items, chunks = a.chunks;
  const int chunks_a = a.chunks_a, lo_a = a.lo_a, hi_a = a.hi_a, lo_b = a.lo_b, hi_b = a.hi_b, head = a.head;
  const int wrap_tok = a.wrap_tok;
  const void* const k_new = a.k_new;
  const void* const v_new = a.v_new;
  asm volatile("" ::"s"(H), "s"(grid), "s"(items), "s"(chunks), "s"(chunks_a), "s"(lo_a), "s"(hi_a),
               "s"(lo_b), "s"(hi_b), "s"(head), "s"(wrap_tok), "s"(k_new), "s"(v_new));
  // Workgroups are dealt to the 8 XCDs in turn; give each XCD a contiguous
  // range of work items, so that the neighbouring chunks whose V^T pieces
  // share 128-byte lines are written through the same L2.
  const int item = (blockIdx.x % 8) * (grid / 8) + blockIdx.x / 8;
  if (item >= items) return;
  const int c = item % chunks;
  const int group = item / chunks;
  int base, lo, hi;
  if (c < chunks_a) {
    base = (lo_a / kWChunk + c) * kWChunk;
    lo = max(base, lo_a);
    hi = min(base + kWChunk, hi_a);
  } else {
    base = (lo_b / kWChunk + (c - chunks_a)) * kWChunk;
    lo = max(base, lo_b);
    hi = min(base + kWChunk, hi_b);
  }
  // token index of slot s (slots of one chunk have consecutive tokens): slots
  // from head on hold tokens 0.., the wrapped range [lo_b, hi_b) (below head)
  // continues with token E - head, E the end of the ring part
  auto token_of = [&](int s) {
    int t = s - head;
    return t < 0 ? t + wrap_tok : t;
  };
  const int piece = tid % kLanesPerRow;
  const int rg = tid / kLanesPerRow;
  const int hh = rg / kSlotGroups;                       // head of this thread's rows
  const int sl0 = (rg % kSlotGroups) * kRowsPerThread;   // first of its 4 slots
  const int h = group * kWHeads + hh;

  // ---- all input loads first
  Raw<KV, EPL> rk[kRowsPerThread], rv[kRowsPerThread];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int s = base + sl0 + i;
#pragma unroll
    for (int w = 0; w < Raw<KV, EPL>::words; ++w) rk[i].w[w] = rv[i].w[w] = 0u;
    if (s >= lo && s < hi && h < H) {
      const size_t off = (static_cast<size_t>(token_of(s)) * H + h) * D + piece * EPL;
      load_raw<KV, EPL>(k_new, off, rk[i]);
      load_raw<KV, EPL>(v_new, off, rv[i]);
    }
  }
  double rev[EPL / 2];
#pragma unroll
  for (int e = 0; e < EPL / 2; ++e) rev[e] = a.rope.rev[piece * (EPL / 2) + e];

  // ---- slot metadata (first head group only)
  if (group == 0 && tid < kWChunk) {
    const int s = base + tid;
    if (s >= lo && s < hi) {
      a.r.slot_pos[s] = a.pos0 + token_of(s);
      a.r.slot_block[s] = a.block_id;
    }
  }
  // position of this thread's first slot: the chunk's slots from lo on hold
  // consecutive tokens (rows outside [lo, hi) are computed but not stored)
  const long long pos_first = static_cast<long long>(a.pos0) + token_of(lo) + (base + sl0 - lo);

  // ---- rows: rotate, quantise, store K; quantise V
  uint32_t vcode[kRowsPerThread][EPL / 4];  // FP8 codes of V (ES == 1)
  float vval[kRowsPerThread][ES == 1 ? 1 : EPL];  // V values (BF16 / F32 rings)
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int s = base + sl0 + i;
    const bool valid = s >= lo && s < hi && h < H;
    float xk[EPL], xv[EPL];
    unpack<KV, EPL>(rk[i], xk);
    unpack<KV, EPL>(rv[i], xv);
    if (a.use_rope) {
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) {
        double r = static_cast<double>(pos_first + i) * rev[e];
        r -= rint(r);
        const float t = static_cast<float>(r);
        const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
        const float x0 = xk[2 * e], x1 = xk[2 * e + 1];
        xk[2 * e] = x0 * cs - x1 * sn;
        xk[2 * e + 1] = x0 * sn + x1 * cs;
      }
    }
    float ks = 0.f, vs = 0.f, krc = 0.f, vrc = 0.f;
    if constexpr (KV == KV_FP8) {
      ks = row_scale<kLanesPerRow, EPL>(xk);
      vs = row_scale<kLanesPerRow, EPL>(xv);
      krc = scale_rcp(ks);
      vrc = scale_rcp(vs);
    }
    if (valid) {
      const size_t srow = static_cast<size_t>(h) * a.r.v_ld + s;
      // rotated keys: direct product; unrotated keys: exact quotient
      if (a.use_rope) store_row<KV, EPL, false>(a.r.k, srow * D + piece * EPL, xk, ks, krc);
      else store_row<KV, EPL, true>(a.r.k, srow * D + piece * EPL, xk, ks, krc);
      if constexpr (KV == KV_FP8) {
        if (piece == 0) {
          a.r.k_scale[srow] = ks;
          a.r.v_scale[srow] = vs;
        }
      }
    }
    if constexpr (KV == KV_FP8) {
      encode_fp8<EPL, true>(xv, vs, vrc, vcode[i]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) vval[i][e] = xv[e];
    }
  }
  // ---- V^T in LDS: row (hh, j) at (hh * D + j) * RS; this thread's 4 slots of
  //      each of its d values j go in as one piece (4 codes, 4 bf16 or 4 floats)
  uint8_t* vrow = vt + (static_cast<size_t>(hh) * D + piece * EPL) * RS + sl0 * ES;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    uint8_t* dst = vrow + e * RS;
    if constexpr (KV == KV_FP8) {
      // byte e % 4 of word e / 4 of each row, gathered into one word
      const int sh = 8 * (e % 4);
      const uint32_t b0 = (vcode[0][e / 4] >> sh) & 0xFFu, b1 = (vcode[1][e / 4] >> sh) & 0xFFu;
      const uint32_t b2 = (vcode[2][e / 4] >> sh) & 0xFFu, b3 = (vcode[3][e / 4] >> sh) & 0xFFu;
      *reinterpret_cast<uint32_t*>(dst) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    } else if constexpr (KV == KV_BF16) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(vval[0][e], vval[1][e]), pack_bf16x2(vval[2][e], vval[3][e]));
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(vval[0][e], vval[1][e], vval[2][e], vval[3][e]);
    }
  }
  __syncthreads();

  // ---- V^T rows -> global, 16-byte pieces
  constexpr int kSlotsPerPiece = 16 / ES;
  constexpr int kPiecesPerRow = kWChunk / kSlotsPerPiece;
  for (int u = tid; u < kWHeads * D * kPiecesPerRow; u += kThreads) {
    const int hq = u / (D * kPiecesPerRow);
    const int rem = u - hq * (D * kPiecesPerRow);
    const int j = rem / kPiecesPerRow, w = rem - j * kPiecesPerRow;
    const int hd = group * kWHeads + hq;
    if (hd >= H) continue;
    const int s0 = base + w * kSlotsPerPiece;
    const uint8_t* src = vt + (static_cast<size_t>(hq) * D + j) * RS + w * 16;
    uint8_t* dst = static_cast<uint8_t*>(a.r.v) + ((static_cast<size_t>(hd) * D + j) * a.r.v_ld + s0) * ES;
    if (s0 >= lo && s0 + kSlotsPerPiece <= hi) {
      const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
      *reinterpret_cast<uint4*>(dst) = make_uint4(s32[0], s32[1], s32[2], s32[3]);
    } else {
      for (int q = 0; q < kSlotsPerPiece; ++q) {
        if (s0 + q >= lo && s0 + q < hi) {
#pragma unroll
          for (int b = 0; b < ES; ++b) dst[q * ES + b] = src[q * ES + b];
        }
      }
    }
  }
}

// FP8 write.  One launch, two kinds of workgroup (uniform per workgroup),
// neither with LDS or a barrier, so that every wave loads, converts and
// stores on its own and loads and stores of different waves overlap as in a
// plain copy:
//  * K workgroups take (token, head) rows in input order, kKRows per group
//    of 16 lanes: rotate, quantise and store each row (one d-byte cache row).
//    The rotation angles depend on the token and the pair only, so a
//    workgroup computes each (token, pair) cosine and sine once, into LDS,
//    while its row loads are in flight (every head of a token shares them);
//  * V workgroups take one head and a 128-slot aligned tile of the written
//    range, 4 consecutive slots x D/16 values per thread; each thread stores,
//    for each of its values, the 4 slots' codes as one word of the V^T row,
//    so a wave's store covers 16 consecutive slots of 16 V^T rows and the
//    workgroup's stores fill whole 128-byte lines (except at the ends of the
//    written range), merged in the L2 of the one XCD the workgroup runs on.
// V workgroups of head 0 also write slot_pos and slot_block.
constexpr int kWThreadsFp8 = 512;
constexpr int kVTile = 128;     // slots per V workgroup
constexpr int kVSlots = 4;      // consecutive slots per thread of a V workgroup
constexpr int kKRows = 2;       // rows per 16-lane group of a K workgroup
constexpr int kKRowsPerWg = kWThreadsFp8 / kLanesPerRow * kKRows;
constexpr int kKTokMax = kKRowsPerWg + 1;  // tokens one K workgroup's rows can span (H >= 1)
static_assert(kWThreadsFp8 / kLanesPerRow * kVSlots == kVTile, "V tile");

template <int D>
__global__ __launch_bounds__(kWThreadsFp8) void cache_write_fp8_kernel(WriteArgs a, int k_wgs) {
  constexpr int EPL = D / kLanesPerRow;  // elements per lane (8 or 4)
  const int tid = threadIdx.x;
  const int H = a.r.H, n_new = a.n_new, head = a.head, wrap_tok = a.wrap_tok;
  const int lo_a = a.lo_a, hi_a = a.hi_a, lo_b = a.lo_b;
  asm volatile("" ::"s"(H), "s"(n_new), "s"(head), "s"(wrap_tok), "s"(lo_a), "s"(hi_a), "s"(lo_b), "s"(k_wgs));
  const int piece = tid % kLanesPerRow;
  const int rg = tid / kLanesPerRow;

  if (static_cast<int>(blockIdx.x) < k_wgs) {
    // ---- K rows: row index t * H + h (token t, head h), input order
    const int n_rows = n_new * H;
    const int row0 = blockIdx.x * kKRowsPerWg + rg * kKRows;
    Raw<KV_FP8, EPL> rk[kKRows];
#pragma unroll
    for (int i = 0; i < kKRows; ++i) {
#pragma unroll
      for (int w = 0; w < Raw<KV_FP8, EPL>::words; ++w) rk[i].w[w] = 0u;
      if (row0 + i < n_rows) load_raw<KV_FP8, EPL>(a.k_new, static_cast<size_t>(row0 + i) * D + piece * EPL, rk[i]);
    }
    // (cos, sin) of every (token, pair) of this workgroup's rows: the angle
    // pos * theta_i reduced in float64 to at most half a revolution, then the
    // hardware sine and cosine (which take revolutions)
    __shared__ float2 cs_tab[kKTokMax * (D / 2)];
    const int wg_row0 = blockIdx.x * kKRowsPerWg;
    const int t_lo = wg_row0 / H;
    if (a.use_rope) {
      const int t_hi = min(wg_row0 + kKRowsPerWg, n_rows) - 1;
      const int n_ang = (t_hi / H - t_lo + 1) * (D / 2);
      for (int i = tid; i < n_ang; i += kWThreadsFp8) {
        const int e = i % (D / 2);
        const long long pos = static_cast<long long>(a.pos0) + t_lo + i / (D / 2);
        double r = static_cast<double>(pos) * a.rope.rev[e];
        r -= rint(r);
        const float tt = static_cast<float>(r);
        cs_tab[i] = make_float2(__builtin_amdgcn_cosf(tt), __builtin_amdgcn_sinf(tt));
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kKRows; ++i) {
      const int row = row0 + i;
      const int t = min(row, n_rows - 1) / H, h = min(row, n_rows - 1) % H;
      float xk[EPL];
      unpack<KV_FP8, EPL>(rk[i], xk);
      if (a.use_rope) {
        const float2* cs_row = cs_tab + (t - t_lo) * (D / 2) + piece * (EPL / 2);
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          const float2 c = cs_row[e];
          const float x0 = xk[2 * e], x1 = xk[2 * e + 1];
          xk[2 * e] = x0 * c.x - x1 * c.y;
          xk[2 * e + 1] = x0 * c.y + x1 * c.x;
        }
      }
      const float ks = row_scale<kLanesPerRow, EPL>(xk);
      const float krc = scale_rcp(ks);
      if (row < n_rows) {
        const int slot = t < hi_a - lo_a ? lo_a + t : lo_b + (t - (hi_a - lo_a));
        const size_t srow = static_cast<size_t>(h) * a.r.v_ld + slot;
        // rotated keys: direct product; unrotated keys: exact quotient
        if (a.use_rope) store_row<KV_FP8, EPL, false>(a.r.k, srow * D + piece * EPL, xk, ks, krc);
        else store_row<KV_FP8, EPL, true>(a.r.k, srow * D + piece * EPL, xk, ks, krc);
        if (piece == 0) a.r.k_scale[srow] = ks;
      }
    }
    return;
  }

  // ---- V tile: head h, slots base .. base + 127 clipped to [lo, hi)
  const int item = blockIdx.x - k_wgs;
  const int h = item % H;
  const int c = item / H;
  int base, lo, hi;
  if (c < a.chunks_a) {
    base = (lo_a / kVTile + c) * kVTile;
    lo = max(base, lo_a);
    hi = min(base + kVTile, hi_a);
  } else {
    base = (lo_b / kVTile + (c - a.chunks_a)) * kVTile;
    lo = max(base, lo_b);
    hi = min(base + kVTile, a.hi_b);
  }
  auto token_of = [&](int sl) {
    int t = sl - head;
    return t < 0 ? t + wrap_tok : t;
  };
  // thread: slots s0 .. s0 + 3, values piece * EPL .. + EPL - 1
  const int s0 = base + kVSlots * rg;
  Raw<KV_FP8, EPL> rv[kVSlots];
#pragma unroll
  for (int i = 0; i < kVSlots; ++i) {
#pragma unroll
    for (int w = 0; w < Raw<KV_FP8, EPL>::words; ++w) rv[i].w[w] = 0u;
    const int sl = s0 + i;
    if (sl >= lo && sl < hi)
      load_raw<KV_FP8, EPL>(a.v_new, (static_cast<size_t>(token_of(sl)) * H + h) * D + piece * EPL, rv[i]);
  }
  if (h == 0 && tid < kVTile) {
    const int sl = base + tid;
    if (sl >= lo && sl < hi) {
      a.r.slot_pos[sl] = a.pos0 + token_of(sl);
      a.r.slot_block[sl] = a.block_id;
    }
  }
  uint32_t code[kVSlots][EPL / 4];
#pragma unroll
  for (int i = 0; i < kVSlots; ++i) {
    float xv[EPL];
    unpack<KV_FP8, EPL>(rv[i], xv);
    const float vs = row_scale<kLanesPerRow, EPL>(xv);
    encode_fp8<EPL, true>(xv, vs, scale_rcp(vs), code[i]);
    const int sl = s0 + i;
    if (piece == 0 && sl >= lo && sl < hi) a.r.v_scale[static_cast<size_t>(h) * a.r.v_ld + sl] = vs;
  }
  // value j = piece * EPL + e of the 4 slots -> one word of V^T row (h, j)
  const bool whole = s0 >= lo && s0 + kVSlots <= hi;
  uint8_t* vrow = static_cast<uint8_t*>(a.r.v) + (static_cast<size_t>(h) * D + piece * EPL) * a.r.v_ld + s0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int sh = 8 * (e % 4);
    const uint32_t b0 = (code[0][e / 4] >> sh) & 0xFFu, b1 = (code[1][e / 4] >> sh) & 0xFFu;
    const uint32_t b2 = (code[2][e / 4] >> sh) & 0xFFu, b3 = (code[3][e / 4] >> sh) & 0xFFu;
    uint8_t* dst = vrow + static_cast<size_t>(e) * a.r.v_ld;
    if (whole) {
      *reinterpret_cast<uint32_t*>(dst) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    } else {
      const uint32_t bytes[4] = {b0, b1, b2, b3};
#pragma unroll
      for (int q = 0; q < kVSlots; ++q)
        if (s0 + q >= lo && s0 + q < hi) dst[q] = static_cast<uint8_t>(bytes[q]);
    }
  }
}

// Delta re-rotation of every occupied row.  A row of K (d elements) is
// handled by LPR lanes with 16 bytes each; a thread takes kRotRows rows whose
// loads are all issued before any of the rows' arithmetic.
constexpr int kRotRows = 2;

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void rerotate_kernel(RingView r, int delta, RopeTable rope) {
  constexpr int ES = Store<KV>::bytes;
  constexpr int EPT = 16 / ES;          // elements per thread
  constexpr int LPR = D / EPT;          // lanes per row
  constexpr int RPB = kThreads / LPR;   // rows per block pass
  const int lane = threadIdx.x % LPR;
  // A wave needs only the d/2 factor pairs: each lane computes pair
  // (its lane index mod d/2) and takes the EPT/2 pairs of its row piece from
  // the lanes that hold them.
  static_assert(D / 2 <= kWave, "one factor pair per lane");
  float c1, s1;
  rope_cs(rope, (threadIdx.x % kWave) % (D / 2), delta, &c1, &s1);
  float cc[EPT / 2], ss[EPT / 2];
#pragma unroll
  for (int e = 0; e < EPT / 2; ++e) {
    cc[e] = __shfl(c1, lane * (EPT / 2) + e, kWave);
    ss[e] = __shfl(s1, lane * (EPT / 2) + e, kWave);
  }
  // head h = blockIdx.y; slots s0 + i * stride of it (no division per row)
  const int h = blockIdx.y;
  const int stride = gridDim.x * RPB;
  for (int s0 = blockIdx.x * RPB + threadIdx.x / LPR; s0 < r.N; s0 += kRotRows * stride) {
    uint4 raw[kRotRows];
    float sc[kRotRows];
    bool live[kRotRows];
#pragma unroll
    for (int i = 0; i < kRotRows; ++i) {
      const int s = s0 + i * stride;
      live[i] = false;
      raw[i] = make_uint4(0u, 0u, 0u, 0u);
      sc[i] = 0.f;
      if (s < r.N) {
        const size_t srow = static_cast<size_t>(h) * r.v_ld + s;
        live[i] = r.slot_block[s] != -1;
        raw[i] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(r.k) + (srow * D + lane * EPT) * ES);
        if constexpr (KV == KV_FP8) sc[i] = r.k_scale[srow];
      }
    }
#pragma unroll
    for (int i = 0; i < kRotRows; ++i) {
      const int s = s0 + i * stride;
      if (s >= r.N) continue;  // whole rows (and so whole lane groups) skip together
      const size_t srow = static_cast<size_t>(h) * r.v_ld + s;
      float x[EPT];
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      if constexpr (KV == KV_FP8) {
        // FP8 rows are rotated in code units (two codes per conversion): the
        // old scale s cancels from the new codes, round(R(c s) / (s max|R c| /
        // 448)) = round(R c / (max|R c| / 448)), and enters only the new
        // scale s max|R c| / 448
#pragma unroll
        for (int e = 0; e < EPT / 4; ++e) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[e]), false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[e]), true);
          x[4 * e] = lo[0];
          x[4 * e + 1] = lo[1];
          x[4 * e + 2] = hi[0];
          x[4 * e + 3] = hi[1];
        }
      } else if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int e = 0; e < EPT / 2; ++e) {
          x[2 * e] = __uint_as_float(w[e] << 16);
          x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) x[e] = __uint_as_float(w[e]);
      }
#pragma unroll
      for (int e = 0; e < EPT / 2; ++e) {
        const float x0 = x[2 * e], x1 = x[2 * e + 1];
        x[2 * e] = x0 * cc[e] - x1 * ss[e];
        x[2 * e + 1] = x0 * ss[e] + x1 * cc[e];
      }
      float nsc = 0.f, rc = 0.f;
      if constexpr (KV == KV_FP8) {
        const float csc = row_scale<LPR, EPT>(x);  // max|R c| / 448
        rc = scale_rcp(csc);
        nsc = csc * sc[i];
      }
      if (!live[i]) continue;  // whole rows skip together (after the row's shuffles)
      store_row<KV, EPT, false>(r.k, srow * D + lane * EPT, x, nsc, rc);  // rotated in float32
      if constexpr (KV == KV_FP8) {
        if (lane == 0) r.k_scale[srow] = nsc;
      }
      if (h == 0 && lane == 0) r.slot_pos[s] += delta;
    }
  }
}

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
  for (size_t i = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * kThreads)
    p[i] = value;
}

RopeTable make_rope(float base, int d) {
  RopeTable t{};
  for (int j = 0; j < d / 2 && j < 64; ++j)
    t.rev[j] = base > 0.f ? std::pow(static_cast<double>(base), -2.0 * j / d) / (2.0 * M_PI) : 0.0;
  return t;
}

hipError_t fill(void* p, size_t bytes, uint32_t value, hipStream_t s) {
  if (!p || bytes == 0) return hipSuccess;
  size_t n = bytes / 4;
  int blocks = static_cast<int>(std::min<size_t>((n + kThreads - 1) / kThreads, 4096));
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(kThreads), 0, s, static_cast<uint32_t*>(p), n,
                     value);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t write_impl(const WriteArgs& a, hipStream_t s) {
  WriteArgs b = a;
  if constexpr (KV == KV_FP8) {
    // V tiles of 128 slots, one head each; K rows in blocks of kKRowsPerWg
    b.chunks_a = (a.hi_a - 1) / kVTile - a.lo_a / kVTile + 1;
    const int chunks_b = a.hi_b > a.lo_b ? (a.hi_b - 1) / kVTile - a.lo_b / kVTile + 1 : 0;
    const int v_wgs = (b.chunks_a + chunks_b) * a.r.H;
    const int k_wgs = (a.n_new * a.r.H + kKRowsPerWg - 1) / kKRowsPerWg;
    hipLaunchKernelGGL((cache_write_fp8_kernel<D>), dim3(k_wgs + v_wgs), dim3(kWThreadsFp8), 0, s, b, k_wgs);
  } else {
    b.grid = (a.items + 7) / 8 * 8;  // a multiple of 8 for the XCD mapping
    hipLaunchKernelGGL((cache_write_kernel<KV, D>), dim3(b.grid), dim3(kThreads), 0, s, b);
  }
  return hipGetLastError();
}

template <int KV, int D>
hipError_t rerotate_impl(const RingView& r, int delta, hipStream_t s) {
  RopeTable t = make_rope(r.rope_base, r.d);
  constexpr int LPR = D / (16 / Store<KV>::bytes);
  constexpr int RPB = kThreads / LPR;
  const int blocks = std::max(1, std::min((r.N + RPB * kRotRows - 1) / (RPB * kRotRows), 4096));
  hipLaunchKernelGGL((rerotate_kernel<KV, D>), dim3(blocks, r.H), dim3(kThreads), 0, s, r, delta, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ring_clear(const RingView& r, hipStream_t s) {
  const size_t es = r.kv == KV_F32 ? 4 : (r.kv == KV_BF16 ? 2 : 1);
  hipError_t e;
  if ((e = fill(r.k, static_cast<size_t>(r.H) * r.v_ld * r.d * es, 0u, s)) != hipSuccess) return e;
  if ((e = fill(r.v, static_cast<size_t>(r.H) * r.d * r.v_ld * es, 0u, s)) != hipSuccess) return e;
  if (r.kv == KV_FP8) {
    if ((e = fill(r.k_scale, static_cast<size_t>(r.H) * r.v_ld * 4, 0u, s)) != hipSuccess) return e;
    if ((e = fill(r.v_scale, static_cast<size_t>(r.H) * r.v_ld * 4, 0u, s)) != hipSuccess) return e;
  }
  if ((e = fill(r.slot_pos, static_cast<size_t>(r.v_ld) * 4, 0u, s)) != hipSuccess) return e;
  return fill(r.slot_block, static_cast<size_t>(r.v_ld) * 4, 0xFFFFFFFFu, s);
}

hipError_t launch_cache_write(const RingView& r, const void* k_new, const void* v_new, int n_new,
                              int head, int pos0, int block_id, hipStream_t s) {
  WriteArgs a{};
  a.r = r;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  a.head = head;
  a.pos0 = pos0;
  a.block_id = block_id;
  // the ring part is slots n_anchor .. E-1; the part of the write past
  // slot E-1 wraps to its first slot
  const int E = r.N - r.n_memory;
  a.lo_a = head;
  a.hi_a = std::min(head + n_new, E);
  a.lo_b = r.n_anchor;
  a.hi_b = head + n_new > E ? r.n_anchor + head + n_new - E : r.n_anchor;
  a.wrap_tok = E - r.n_anchor;
  a.chunks_a = (a.hi_a - 1) / kWChunk - a.lo_a / kWChunk + 1;
  const int chunks_b = a.hi_b > a.lo_b ? (a.hi_b - 1) / kWChunk - a.lo_b / kWChunk + 1 : 0;
  a.use_rope = r.rope_base > 0.f;
  a.rope = make_rope(r.rope_base, r.d);
  a.chunks = a.chunks_a + chunks_b;
  a.items = a.chunks * ((r.H + kWHeads - 1) / kWHeads);
  switch (r.kv * 1000 + r.d) {
    case KV_FP8 * 1000 + 128: return write_impl<KV_FP8, 128>(a, s);
    case KV_FP8 * 1000 + 64: return write_impl<KV_FP8, 64>(a, s);
    case KV_BF16 * 1000 + 128: return write_impl<KV_BF16, 128>(a, s);
    case KV_BF16 * 1000 + 64: return write_impl<KV_BF16, 64>(a, s);
    case KV_F32 * 1000 + 128: return write_impl<KV_F32, 128>(a, s);
    case KV_F32 * 1000 + 64: return write_impl<KV_F32, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rerotate(const RingView& r, int delta, hipStream_t s) {
  switch (r.kv * 1000 + r.d) {
    case KV_FP8 * 1000 + 128: return rerotate_impl<KV_FP8, 128>(r, delta, s);
    case KV_FP8 * 1000 + 64: return rerotate_impl<KV_FP8, 64>(r, delta, s);
    case KV_BF16 * 1000 + 128: return rerotate_impl<KV_BF16, 128>(r, delta, s);
    case KV_BF16 * 1000 + 64: return rerotate_impl<KV_BF16, 64>(r, delta, s);
    case KV_F32 * 1000 + 128: return rerotate_impl<KV_F32, 128>(r, delta, s);
    case KV_F32 * 1000 + 64: return rerotate_impl<KV_F32, 64>(r, delta, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rc
