// Ring-cache write, delta re-rotation and clear kernels (gfx950).
//
// The write moves each chunk's new K and V into the ring once, applying RoPE
// to K and FP8 quantisation to both at write time, and the re-rotation moves
// every cached key to new positions by a delta rotation (Runway Characters,
// abstract).  Both are HBM-bound: each byte of input is read once and each
// byte of the cache written once.
//
// Write layout: the written range [head, head + n) mod N is cut into at most
// two linear slot ranges, and each range into 64-slot chunks aligned to
// multiples of 64.  One workgroup handles one chunk for a group of heads:
//  * cos/sin of every (slot, pair) of the chunk go to LDS once and are reused
//    for every head of the group;
//  * a K row (one token of one head, d elements) is handled by 16 lanes, so a
//    pass of 256 threads covers 16 slots; each lane stores d/16 contiguous
//    elements and the 16 lanes a whole contiguous cache row;
//  * V is quantised the same way, transposed through LDS and stored to the
//    [H][d][v_ld] layout as 16-byte pieces of each row (64-slot chunks start
//    on a multiple of 64 and v_ld is a multiple of 64, so pieces are aligned).
#include <algorithm>
#include <cmath>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerPass = kThreads / kLanesPerRow;

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
  int heads_per_group;
  int use_rope;
  RopeTable rope;
};

// Loads EPL input elements of one (token, head) row, as float.
template <int KV, int EPL>
__device__ __forceinline__ void load_row(const void* base, size_t elem_off, float* x) {
  if constexpr (KV == KV_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      float4 t = p[i];
      x[4 * i] = t.x;
      x[4 * i + 1] = t.y;
      x[4 * i + 2] = t.z;
      x[4 * i + 3] = t.w;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + elem_off;
    if constexpr (EPL == 8) {
      uint4 t = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      uint2 t = *reinterpret_cast<const uint2*>(p);
      uint32_t w[2] = {t.x, t.y};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
}

// x / scale rounded to float32 with round-to-odd, so that the FP8 conversion
// that follows (round to nearest even) yields the correctly rounded code of
// the exact quotient.  A plain float32 quotient can land exactly on a
// midpoint between two FP8 codes when the exact quotient lies just beside it
// (common: x and the absmax carry 8 significant bits, so 448 x / absmax is
// often a short fraction, while scale = absmax / 448 is rounded), and the
// conversion's tie-break would then round the wrong way.  Round-to-odd keeps
// the "inexact" information in the last bit (float32 has 20 more bits than
// e4m3), the classical remedy for double rounding.  A zero scale gives 0.
__device__ __forceinline__ float qdiv(float x, float scale) {
  if (!(scale > 0.f)) return 0.f;
  const float q = x / scale;             // correctly rounded
  const float r = fmaf(-q, scale, x);    // exact remainder x - q * scale
  if (r == 0.f || q == 0.f) return q;
  uint32_t u = __float_as_uint(q);
  if ((r > 0.f) != (q > 0.f)) u -= 1;    // exact quotient is nearer zero: truncate
  return __uint_as_float(u | 1u);        // inexact: force the last bit to 1
}

// Stores EPL values of a K row: FP8 codes (given the row's scale), bf16 or
// float32.
template <int KV, int EPL>
__device__ __forceinline__ void store_row(void* base, size_t elem_off, const float* x, float sc) {
  if constexpr (KV == KV_FP8) {
    uint8_t* p = static_cast<uint8_t*>(base) + elem_off;
    if constexpr (EPL == 8) {
      uint2 w;
      w.x = cvt_fp8x4(qdiv(x[0], sc), qdiv(x[1], sc), qdiv(x[2], sc), qdiv(x[3], sc));
      w.y = cvt_fp8x4(qdiv(x[4], sc), qdiv(x[5], sc), qdiv(x[6], sc), qdiv(x[7], sc));
      *reinterpret_cast<uint2*>(p) = w;
    } else {
      *reinterpret_cast<uint32_t*>(p) = cvt_fp8x4(qdiv(x[0], sc), qdiv(x[1], sc), qdiv(x[2], sc), qdiv(x[3], sc));
    }
  } else if constexpr (KV == KV_BF16) {
    uint16_t* p = static_cast<uint16_t*>(base) + elem_off;
    if constexpr (EPL == 8) {
      uint4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
      *reinterpret_cast<uint4*>(p) = w;
    } else {
      uint2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *reinterpret_cast<uint2*>(p) = w;
    }
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) p[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  }
}

// Row absmax over the 16 lanes of a row -> scale = max|x| / 448 in float32
// (IEEE division); a zero row gives 0.
template <int EPL>
__device__ __forceinline__ float row_scale(const float* x) {
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
  a = group_max<kLanesPerRow>(a);
  return a / 448.0f;
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(WriteArgs a) {
  constexpr int EPL = D / kLanesPerRow;
  constexpr int ES = Store<KV>::bytes;
  __shared__ float2 cs[kChunk][D / 2];
  __shared__ __attribute__((aligned(16))) uint8_t vt[D * kChunk * ES];

  const int tid = threadIdx.x;
  const int N = a.r.N;
  const int c = blockIdx.x;
  int base, lo, hi;
  if (c < a.chunks_a) {
    base = (a.lo_a / kChunk + c) * kChunk;
    lo = max(base, a.lo_a);
    hi = min(base + kChunk, a.hi_a);
  } else {
    base = (a.lo_b / kChunk + (c - a.chunks_a)) * kChunk;
    lo = max(base, a.lo_b);
    hi = min(base + kChunk, a.hi_b);
  }
  auto token_of = [&](int s) {
    int t = s - a.head;
    return t < 0 ? t + N : t;
  };

  if (a.use_rope) {
    for (int e = tid; e < kChunk * (D / 2); e += kThreads) {
      int r = e / (D / 2), j = e - r * (D / 2);
      int s = base + r;
      float cc = 1.f, ss = 0.f;
      if (s >= lo && s < hi) rope_cs(a.rope, j, static_cast<long long>(a.pos0) + token_of(s), &cc, &ss);
      cs[r][j] = make_float2(cc, ss);
    }
    __syncthreads();
  }

  if (blockIdx.y == 0 && tid < kChunk) {
    int s = base + tid;
    if (s >= lo && s < hi) {
      a.r.slot_pos[s] = a.pos0 + token_of(s);
      a.r.slot_block[s] = a.block_id;
    }
  }

  const int lane16 = tid % kLanesPerRow;
  const int h0 = blockIdx.y * a.heads_per_group;
  const int h1 = min(h0 + a.heads_per_group, a.r.H);
  const int H = a.r.H;
  for (int h = h0; h < h1; ++h) {
#pragma unroll
    for (int p = 0; p < kChunk / kRowsPerPass; ++p) {
      const int r = p * kRowsPerPass + tid / kLanesPerRow;
      const int s = base + r;
      const bool valid = s >= lo && s < hi;
      float xk[EPL], xv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) xk[e] = xv[e] = 0.f;
      if (valid) {
        const size_t off = (static_cast<size_t>(token_of(s)) * H + h) * D + lane16 * EPL;
        load_row<KV, EPL>(a.k_new, off, xk);
        load_row<KV, EPL>(a.v_new, off, xv);
      }
      if (a.use_rope) {
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          float2 t = cs[r][lane16 * (EPL / 2) + e];
          float x0 = xk[2 * e], x1 = xk[2 * e + 1];
          xk[2 * e] = x0 * t.x - x1 * t.y;
          xk[2 * e + 1] = x0 * t.y + x1 * t.x;
        }
      }
      float ks = 0.f, vs = 0.f;
      if constexpr (KV == KV_FP8) {
        ks = row_scale<EPL>(xk);
        vs = row_scale<EPL>(xv);
      }
      if (valid) {
        const size_t row = static_cast<size_t>(h) * a.r.v_ld + s;
        store_row<KV, EPL>(a.r.k, row * D + lane16 * EPL, xk, ks);
        if constexpr (KV == KV_FP8) {
          if (lane16 == 0) {
            a.r.k_scale[row] = ks;
            a.r.v_scale[row] = vs;
          }
        }
      }
      // V to LDS, transposed [D][kChunk]
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = lane16 * EPL + e;
        if constexpr (KV == KV_FP8) {
          if (e % 2 == 0) {
            const uint32_t w =
                static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(qdiv(xv[e], vs), qdiv(xv[e + 1], vs), 0, false));
            vt[j * kChunk + r] = static_cast<uint8_t>(w & 0xFF);
            vt[(j + 1) * kChunk + r] = static_cast<uint8_t>((w >> 8) & 0xFF);
          }
        } else if constexpr (KV == KV_BF16) {
          reinterpret_cast<uint16_t*>(vt)[j * kChunk + r] = f32_to_bf16(xv[e]);
        } else {
          reinterpret_cast<float*>(vt)[j * kChunk + r] = xv[e];
        }
      }
    }
    __syncthreads();
    // transposed V rows -> global, 16-byte pieces
    constexpr int kSlotsPerPiece = 16 / ES;
    constexpr int kPiecesPerRow = kChunk / kSlotsPerPiece;
    for (int u = tid; u < D * kPiecesPerRow; u += kThreads) {
      const int j = u / kPiecesPerRow, w = u - j * kPiecesPerRow;
      const int s0 = base + w * kSlotsPerPiece;
      const uint8_t* src = vt + (j * kChunk + w * kSlotsPerPiece) * ES;
      uint8_t* dst = static_cast<uint8_t*>(a.r.v) +
                     ((static_cast<size_t>(h) * D + j) * a.r.v_ld + s0) * ES;
      if (s0 >= lo && s0 + kSlotsPerPiece <= hi) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int q = 0; q < kSlotsPerPiece; ++q) {
          if (s0 + q >= lo && s0 + q < hi) {
#pragma unroll
            for (int b = 0; b < ES; ++b) dst[q * ES + b] = src[q * ES + b];
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int KV, int D>
__global__ __launch_bounds__(kThreads) void rerotate_kernel(RingView r, int delta, RopeTable rope) {
  constexpr int EPL = D / kLanesPerRow;
  const int lane16 = threadIdx.x % kLanesPerRow;
  float cc[EPL / 2], ss[EPL / 2];
#pragma unroll
  for (int e = 0; e < EPL / 2; ++e) rope_cs(rope, lane16 * (EPL / 2) + e, delta, &cc[e], &ss[e]);
  const int rows = r.H * r.N;
  for (int row = blockIdx.x * kRowsPerPass + threadIdx.x / kLanesPerRow; row < rows;
       row += gridDim.x * kRowsPerPass) {
    const int h = row / r.N;
    const int s = row - h * r.N;
    if (r.slot_block[s] == -1) continue;  // the 16 lanes of a row branch together
    const size_t srow = static_cast<size_t>(h) * r.v_ld + s;
    const size_t off = srow * D + lane16 * EPL;
    float x[EPL];
    if constexpr (KV == KV_FP8) {
      const float sc = r.k_scale[srow];
      const uint8_t* p = static_cast<const uint8_t*>(r.k) + off;
      uint32_t w[EPL / 4];
      if constexpr (EPL == 8) {
        uint2 t = *reinterpret_cast<const uint2*>(p);
        w[0] = t.x;
        w[1] = t.y;
      } else {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = fp8_to_f32(w[e / 4], e % 4) * sc;
    } else {
      load_row<KV, EPL>(r.k, off, x);
    }
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) {
      float x0 = x[2 * e], x1 = x[2 * e + 1];
      x[2 * e] = x0 * cc[e] - x1 * ss[e];
      x[2 * e + 1] = x0 * ss[e] + x1 * cc[e];
    }
    float sc = 0.f;
    if constexpr (KV == KV_FP8) sc = row_scale<EPL>(x);
    store_row<KV, EPL>(r.k, off, x, sc);
    if constexpr (KV == KV_FP8) {
      if (lane16 == 0) r.k_scale[srow] = sc;
    }
    if (h == 0 && lane16 == 0) r.slot_pos[s] += delta;
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
hipError_t write_impl(const WriteArgs& a, int chunks, int groups, hipStream_t s) {
  hipLaunchKernelGGL((cache_write_kernel<KV, D>), dim3(chunks, groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t rerotate_impl(const RingView& r, int delta, hipStream_t s) {
  RopeTable t = make_rope(r.rope_base, r.d);
  const int rows = r.H * r.N;
  int blocks = std::min((rows + kRowsPerPass - 1) / kRowsPerPass, 4096);
  hipLaunchKernelGGL((rerotate_kernel<KV, D>), dim3(blocks), dim3(kThreads), 0, s, r, delta, t);
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
  a.lo_a = head;
  a.hi_a = std::min(head + n_new, r.N);
  a.lo_b = 0;
  a.hi_b = head + n_new > r.N ? head + n_new - r.N : 0;
  a.chunks_a = (a.hi_a - 1) / kChunk - a.lo_a / kChunk + 1;
  const int chunks_b = a.hi_b > 0 ? (a.hi_b - 1) / kChunk + 1 : 0;
  a.use_rope = r.rope_base > 0.f;
  a.rope = make_rope(r.rope_base, r.d);
  // Heads per workgroup: enough workgroups to cover the chip, and the
  // chunk's cos/sin table reused over the group.
  const int chunks = a.chunks_a + chunks_b;
  int hpg = 1;
  while (hpg < r.H && chunks * ((r.H + 2 * hpg - 1) / (2 * hpg)) >= 512) hpg *= 2;
  a.heads_per_group = hpg;
  const int groups = (r.H + hpg - 1) / hpg;
  switch (r.kv * 1000 + r.d) {
    case KV_FP8 * 1000 + 128: return write_impl<KV_FP8, 128>(a, chunks, groups, s);
    case KV_FP8 * 1000 + 64: return write_impl<KV_FP8, 64>(a, chunks, groups, s);
    case KV_BF16 * 1000 + 128: return write_impl<KV_BF16, 128>(a, chunks, groups, s);
    case KV_BF16 * 1000 + 64: return write_impl<KV_BF16, 64>(a, chunks, groups, s);
    case KV_F32 * 1000 + 128: return write_impl<KV_F32, 128>(a, chunks, groups, s);
    case KV_F32 * 1000 + 64: return write_impl<KV_F32, 64>(a, chunks, groups, s);
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
