// Fused QKV projection and ring-cache write (gfx950).
//
// Runway Characters (abstract) serves its model with FP8 GEMMs and writes
// each chunk's keys and values into the ring cache once, rotated and
// quantised at write time.  Here the projection [q | k | v] = x W^T runs on
// the FP8 matrix cores and its epilogue does the cache write directly: k and
// v never exist in HBM in any other form than their cached FP8 codes.
//
//  * xquant_kernel: one workgroup per token quantises x (bf16) to
//    FP8 with scale = max|x| / 448 and correctly rounded codes (the cache's
//    rule), stored in 64-byte k slices ([C / 64][token][64]).
//  * qkv_proj_kernel: a workgroup computes 384 tokens x 128 output columns
//    (one head of q, k or v) with 12 waves, three per SIMD; wave w owns
//    tokens 32w .. 32w+31 and all 128 columns (4 MFMA blocks), so every
//    (token, head) row of the result lies in one wave.  At the streaming
//    shape (757 tokens, 3 x 40 heads) that is 240 workgroups: one round on
//    256 CUs.  k steps of 64 bytes: the x tile (384 rows) and the W tile
//    (128 rows) of a step move by direct-to-LDS loads (no registers) into
//    four stages, three steps ahead of use, rows swizzled in 16-byte chunks
//    so that the 32 rows a wave reads together spread over the banks.  The
//    x slice of a step is contiguous in the workspace, so its loads fetch
//    whole 128-byte lines (the L2 request rate, not its bandwidth, is what
//    these loads run into).
//  * the products are formed as W x^T, so that a lane owns one token: lane
//    (n, g) of a wave holds, for its token, 64 of the head's 128 output
//    columns in runs of 4 (the other 64 sit in lane n + 32).
//  * epilogue: values = acc * s_x * s_w; q is rounded to bf16 and stored
//    (unrotated: the attention rotates its queries); k is rotated by RoPE
//    (each pair inside one lane), and k and v are quantised per (token,
//    head) -- absmax over the lane's 64 values and its partner's -- and
//    stored into the ring at the slots of the write: codes packed 4 to a
//    word for k, v transposed with 32 consecutive slots per store, one
//    scale per token.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

constexpr int kPT = 384;             // tokens per workgroup tile
constexpr int kPN = 128;             // output columns per workgroup tile (one head, d = 128)
constexpr int kPK = 64;              // k bytes per step (one FP8 MFMA deep)
constexpr int kPWaves = 12;          // wave w: tokens 32 w .. 32 w + 31, all 128 columns
constexpr int kPThreads = kPWaves * kWave;
constexpr int kABytes = kPT * kPK;   // x tile of a step, 24 KB
constexpr int kBBytes = kPN * kPK;   // W tile of a step, 8 KB
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kLoads = kStageBytes / 1024;  // 1 KB direct-to-LDS loads per step (32)
constexpr int kDmaWaves = 8;                // waves 0..7 issue them, kDma each
constexpr int kDma = kLoads / kDmaWaves;
static_assert(kLoads % kDmaWaves == 0 && kDmaWaves <= kPWaves, "load split");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void glb_void;
typedef __attribute__((address_space(3))) void lds_void;

// 64-byte rows of 4 chunks: chunk c of row r sits at chunk c ^ ((r >> 2) & 3),
// so that the 32 rows a wave reads together spread over the LDS banks.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int tile_addr(int r, int c) { return r * kPK + ((c ^ swz(r)) << 4); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// vmcnt <= N and every LDS read of this wave returned
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct ProjArgs {
  RingView r;
  const uint16_t* x;      // [n][C] bf16
  const uint8_t* w;       // [3 H 128][C] e4m3
  const float* w_scale;   // [3 H 128]
  uint8_t* xq;            // [C / 64][n_pad][64] workspace: 64-byte k slices, token-major
  float* xs;              // [n_pad]
  uint16_t* q_out;        // [n][H][128] bf16
  int n, n_pad, C, pos0, block_id, head, E;
  int m_tiles, items, remap;
  int use_rope;
  RopeTable rope;
};

__global__ __launch_bounds__(256) void xquant_kernel(ProjArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const bool ok = t < a.n;
  const uint16_t* row = a.x + static_cast<size_t>(ok ? t : 0) * a.C;
  float m = 0.f;
  for (int c = tid * 8; c < a.C; c += 256 * 8) {
    const v4u w = *reinterpret_cast<const v4u*>(row + c);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[k] << 16)), fabsf(__uint_as_float(w[k] & 0xFFFF0000u))));
  }
  m = group_max<kWave>(m);
  if (tid % kWave == 0) red[tid / kWave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = ok ? div448(m) : 0.f;
  const float rcp = scale_rcp(sc);
  uint8_t* out = a.xq + static_cast<size_t>(t) * kPK;
  for (int c = tid * 8; c < a.C; c += 256 * 8) {
    const v4u w = ok ? *reinterpret_cast<const v4u*>(row + c) : v4u{0u, 0u, 0u, 0u};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = qdiv_rto(__uint_as_float(w[k] << 16), sc, rcp);
      v[2 * k + 1] = qdiv_rto(__uint_as_float(w[k] & 0xFFFF0000u), sc, rcp);
    }
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(c / kPK) * a.n_pad * kPK + c % kPK) =
        make_uint2(cvt_fp8x4(v[0], v[1], v[2], v[3]), cvt_fp8x4(v[4], v[5], v[6], v[7]));
  }
  if (tid == 0) a.xs[t] = sc;
}

// Slot of token t of the write (consecutive from head, wrapping from E to A).
__device__ __forceinline__ int write_slot(const ProjArgs& a, int t) {
  const int s = a.head + t;
  return s < a.E ? s : a.r.n_anchor + (s - a.E);
}

__global__ __launch_bounds__(kPThreads) void qkv_proj_kernel(ProjArgs a) {
  // four stages of (x tile, W tile), each its own object: the compiler then
  // sees that reading one stage does not wait for loads into the others
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStageBytes];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 31, g = lane >> 5;
  int item = blockIdx.x;
  if (a.remap) item = (item % 8) * (a.items / 8) + item / 8;  // a W tile's token tiles on one XCD
  const int mt = item % a.m_tiles, nt = item / a.m_tiles;
  const int HD = a.r.H * kPN;
  const int col0 = nt * kPN;         // first W row (output column) of the tile
  const int which = col0 / HD;       // 0 q, 1 k, 2 v
  const int h = (col0 % HD) / kPN;
  const int ttok = mt * kPT;         // first token of the tile
  const int C = a.C, S = C / kPK;
  // the epilogue's factors, fetched now so that their latency hides behind
  // the first loads, and parked in LDS: the tile's token scales, column
  // scales and RoPE frequencies
  __shared__ __attribute__((aligned(16))) float s_xs[kPT];
  __shared__ __attribute__((aligned(16))) float s_wsc[kPN];
  __shared__ __attribute__((aligned(16))) double s_rev[kPN / 2];
  const float xs_t = a.xs[ttok + tid % kPT];
  const float wsc = a.w_scale[col0 + tid % kPN];
  const double rev = a.rope.rev[tid % (kPN / 2)];

  // direct-to-LDS loads: 1 KB block q of a stage (x rows 0..383, then W rows
  // 0..127, 4 chunks of 16 bytes a row) is loaded by wave q % 8; its lane l
  // fills LDS chunk p = 64 q + l, which holds global chunk (p % 4) ^ swz(row)
  // of row p / 4.  (32 loads do not split evenly over 12 waves; a wave either
  // issues 4 or none, so that no step branches on it.)
  // (whether block q holds x or W rows is uniform over the wave).  The x
  // slice of a step is one contiguous run of the workspace, so its loads
  // fetch whole 128-byte lines.
  const uint8_t* xbase = a.xq + static_cast<size_t>(ttok) * kPK;
  const size_t xstep = static_cast<size_t>(a.n_pad) * kPK;
  const uint8_t* wbase = a.w + static_cast<size_t>(col0) * C;
  uint32_t off[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int p = (j * kDmaWaves + wave % kDmaWaves) * kWave + lane;
    const bool is_x = p < kPT * 4;
    const int r = is_x ? p >> 2 : (p >> 2) - kPT;
    off[j] = static_cast<uint32_t>(r) * (is_x ? kPK : C) + (((p & 3) ^ swz(r)) << 4);
  }
  auto dma_src = [&](int j, int s) {
    const bool is_x = (j * kDmaWaves + wave % kDmaWaves) * kWave < kPT * 4;
    return (is_x ? xbase + s * xstep : wbase + static_cast<size_t>(s) * kPK) + off[j];
  };

  v16f acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = v16f{};
  // operands of one step (64 bytes of k): this wave's 32 x rows and the 128 W rows
  struct Frag {
    v8i xa, wb[4];
  };
  auto load = [&](const uint8_t* st, Frag& f) {
    const int r = 32 * wave + n;
    const v4i lo = *reinterpret_cast<const v4i*>(st + tile_addr(r, 2 * g));
    const v4i hi = *reinterpret_cast<const v4i*>(st + tile_addr(r, 2 * g + 1));
    f.xa = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int rw = 32 * b + n;
      const v4i wl = *reinterpret_cast<const v4i*>(st + kABytes + tile_addr(rw, 2 * g));
      const v4i wh = *reinterpret_cast<const v4i*>(st + kABytes + tile_addr(rw, 2 * g + 1));
      f.wb[b] = v8i{wl.x, wl.y, wl.z, wl.w, wh.x, wh.y, wh.z, wh.w};
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.wb[b], f.xa, acc[b], 0, 0, 0, 0, 0, 0);
  };
  // step s: wait for this thread's loads of step s (those of s + 1 and s + 2
  // may stay in flight) and for its reads of step s - 1, barrier (all loads
  // of s visible; every wave is done with the stage of s - 1), load step
  // s + 3 into that stage, read the operands of s while those of s - 1
  // multiply.  Before step 0 the held operands are zero codes, whose products
  // add exactly nothing; those of the last step multiply after the loop.
  Frag f0, f1;
  f1.xa = v8i{};
#pragma unroll
  for (int b = 0; b < 4; ++b) f1.wb[b] = v8i{};
  auto park = [&]() {
    if (tid < kPT) s_xs[tid] = xs_t;
    if (tid < kPN) s_wsc[tid] = wsc;
    if (tid < kPN / 2) s_rev[tid] = rev;
  };
  auto main_loop = [&](auto loads) {
    constexpr int L = decltype(loads)::value;
    auto issue = [&](uint8_t* st, int s) {  // past the end, the last step is reloaded (nobody reads it)
      const int ss = min(s, S - 1);
#pragma unroll
      for (int j = 0; j < L; ++j)
        __builtin_amdgcn_global_load_lds((glb_void*)dma_src(j, ss),
                                         (lds_void*)(st + (j * kDmaWaves + wave % kDmaWaves) * 1024), 16, 0, 0);
    };
    auto step = [&](uint8_t* cur, uint8_t* free_st, int s, Frag& fn, const Frag& fp) {
      wait_vm_lds<2 * L>();
      bare_barrier();
      issue(free_st, s + 3);
      load(cur, fn);
      mma(fp);
      __builtin_amdgcn_sched_barrier(0);
    };
    issue(st0, 0);
    issue(st1, 1);
    issue(st2, 2);
    park();
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      step(st0, st3, s, f0, f1);
      step(st1, st0, s + 1, f1, f0);
      step(st2, st1, s + 2, f0, f1);
      step(st3, st2, s + 3, f1, f0);
    }
    // S is even (C is a multiple of 128): the tail has 0 or 2 steps
    if (s < S) {
      step(st0, st3, s, f0, f1);
      step(st1, st0, s + 1, f1, f0);
    }
  };
  if (wave < kDmaWaves)
    main_loop(std::integral_constant<int, kDma>{});
  else
    main_loop(std::integral_constant<int, 0>{});
  mma(f1);
  wait_vm<0>();
  __syncthreads();
  const float sx = s_xs[32 * wave + n];

  // ---- epilogue.  The products were formed as W x^T, so lane (n, g) holds
  //      token tok = tok0 + n, and its element e of column block b is output
  //      column 32 b + 8 (e / 4) + 4 g + e % 4: runs of 4 columns, the two
  //      lanes of a token together covering all 128.
  const int tok0 = ttok + 32 * wave;
  const int tok = tok0 + n;
  const bool live = tok < a.n;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 w4 = *reinterpret_cast<const float4*>(s_wsc + 32 * b + 8 * j + 4 * g);
      acc[b][4 * j + 0] *= sx * w4.x;
      acc[b][4 * j + 1] *= sx * w4.y;
      acc[b][4 * j + 2] *= sx * w4.z;
      acc[b][4 * j + 3] *= sx * w4.w;
    }
  // rows of q and k are staged through LDS (8 KB a wave, in the stages the
  // loop no longer needs) so that each store writes whole 128-byte lines; 16-
  // byte chunks of a row are swizzled against bank conflicts
  uint8_t* stage = (wave < 4 ? st0 : wave < 8 ? st1 : st2) + (wave & 3) * 8192;
  if (which == 0) {  // q: bf16, row-major [token][h][128]: 256-byte rows
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(stage + n * 256 + (((4 * b + j) ^ (n & 15)) << 4) + 8 * g) =
            make_uint2(pack_bf16x2(acc[b][4 * j], acc[b][4 * j + 1]), pack_bf16x2(acc[b][4 * j + 2], acc[b][4 * j + 3]));
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4), ch = lane & 15;
      const v4u v = *reinterpret_cast<const v4u*>(stage + row * 256 + ((ch ^ (row & 15)) << 4));
      if (tok0 + row < a.n)
        *reinterpret_cast<v4u*>(a.q_out + (static_cast<size_t>(tok0 + row) * a.r.H + h) * kPN + 8 * ch) = v;
    }
    return;
  }
  if (which == 1 && a.use_rope) {  // k: rotate pairs (2p, 2p + 1), both in this lane
    const long long pos = static_cast<long long>(a.pos0) + tok;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double2 rv = *reinterpret_cast<const double2*>(s_rev + 16 * b + 4 * j + 2 * g);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float c, sn;
          rope_cs_hw(q ? rv.y : rv.x, pos, &c, &sn);
          const float x0 = acc[b][4 * j + 2 * q], x1 = acc[b][4 * j + 2 * q + 1];
          acc[b][4 * j + 2 * q] = fmaf(-x1, sn, x0 * c);
          acc[b][4 * j + 2 * q + 1] = fmaf(x0, sn, x1 * c);
        }
      }
  }
  // per (token, head) scale: absmax over this lane's 64 values and its partner's
  float m = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(acc[b][e]));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  const float sc = div448(m), rc = scale_rcp(sc);
  uint32_t codes[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      codes[b][j] = cvt_fp8x4(qdiv_rto(acc[b][4 * j], sc, rc), qdiv_rto(acc[b][4 * j + 1], sc, rc),
                              qdiv_rto(acc[b][4 * j + 2], sc, rc), qdiv_rto(acc[b][4 * j + 3], sc, rc));
  const size_t hv = static_cast<size_t>(h) * a.r.v_ld;
  if (which == 1) {  // k rows [h][slot][128]: word (b, j) of the lane is 4-byte
    // piece 2 (j % 2) + g of 16-byte chunk 2 b + j / 2
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint32_t*>(stage + n * kPN + (((2 * b + (j >> 1)) ^ ((n >> 1) & 7)) << 4) +
                                     4 * (2 * (j & 1) + g)) = codes[b][j];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3), ch = lane & 7;
      const v4u v = *reinterpret_cast<const v4u*>(stage + row * kPN + ((ch ^ ((row >> 1) & 7)) << 4));
      if (tok0 + row < a.n)
        *reinterpret_cast<v4u*>(static_cast<uint8_t*>(a.r.k) + (hv + write_slot(a, tok0 + row)) * kPN + 16 * ch) = v;
    }
  }
  if (!live) return;
  const int sl = write_slot(a, tok);
  if (g == 0) (which == 1 ? a.r.k_scale : a.r.v_scale)[hv + sl] = sc;
  if (which == 2) {  // v transposed [h][col][slot]: the 32 lanes of one g write 32
    // consecutive slots of a column row per store
    uint8_t* dst = static_cast<uint8_t*>(a.r.v) + static_cast<size_t>(h) * kPN * a.r.v_ld + sl;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[static_cast<size_t>(32 * b + 8 * j + 4 * g + i) * a.r.v_ld] = static_cast<uint8_t>(codes[b][j] >> (8 * i));
    if (h == 0 && g == 0) {  // slot metadata, once per token
      a.r.slot_pos[sl] = a.pos0 + tok;
      a.r.slot_block[sl] = a.block_id;
    }
  }
}

}  // namespace

size_t qkv_workspace_bytes(int n, int C) {
  const size_t n_pad = static_cast<size_t>((n + kPT - 1) / kPT) * kPT;
  return (n_pad * C + n_pad * 4 + 255) / 256 * 256;
}

hipError_t launch_qkv_project_write(const RingView& r, const void* x, int n, int C, const uint8_t* w,
                                    const float* w_scale, int head, int pos0, int block_id, void* q_out,
                                    void* workspace, hipStream_t s) {
  ProjArgs a{};
  a.r = r;
  a.x = static_cast<const uint16_t*>(x);
  a.w = w;
  a.w_scale = w_scale;
  a.n = n;
  a.n_pad = (n + kPT - 1) / kPT * kPT;
  a.C = C;
  a.xq = static_cast<uint8_t*>(workspace);
  a.xs = reinterpret_cast<float*>(a.xq + static_cast<size_t>(a.n_pad) * C);
  a.q_out = static_cast<uint16_t*>(q_out);
  a.pos0 = pos0;
  a.block_id = block_id;
  a.head = head;
  a.E = r.N - r.n_memory;
  a.m_tiles = a.n_pad / kPT;
  a.items = a.m_tiles * 3 * r.H;
  a.remap = a.items % 8 == 0 ? 1 : 0;
  a.use_rope = r.rope_base > 0.f;
  for (int j = 0; j < kPN / 2; ++j)
    a.rope.rev[j] = a.use_rope ? std::pow(static_cast<double>(r.rope_base), -2.0 * j / kPN) / (2.0 * M_PI) : 0.0;
  hipLaunchKernelGGL(xquant_kernel, dim3(a.n_pad), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qkv_proj_kernel, dim3(a.items), dim3(kPThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rc
