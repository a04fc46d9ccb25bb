// Fused QKV projection and ring-cache write (gfx950).
//
// Runway Characters (abstract) serves its model with FP8 GEMMs and writes
// each chunk's keys and values into the ring cache once, rotated and
// quantised at write time.  Here the projection [q | k | v] = x W^T runs on
// the FP8 matrix cores and its epilogue does the cache write directly: k and
// v never exist in HBM in any other form than their cached FP8 codes.
//
//  * xquant_kernel: one workgroup per token quantises x (bf16) to FP8 with
//    scale = max|x| / 448 and correctly rounded codes (the cache's rule).
//  * qkv_proj_kernel: a workgroup computes 256 tokens x 128 output columns
//    (one head of q, k or v) with 8 waves, two per SIMD; wave w owns tokens
//    32w .. 32w+31 and all 128 columns (4 MFMA blocks), so every
//    (token, head) row of the result lies in one wave.  k steps of 128
//    bytes: the x tile (256 rows) and the W tile (128 rows) of a step move by
//    direct-to-LDS loads (no registers) into three stages, two steps ahead
//    of use, rows swizzled in 16-byte chunks so that the 32 rows a wave reads
//    together spread over the banks.
//  * epilogue: values = acc * s_x * s_w; q is rounded to bf16 and stored
//    (unrotated: the attention rotates its queries); k is rotated by RoPE
//    (pairs sit in neighbouring lanes), and k and v are quantised per
//    (token, head) -- absmax over the row's 32 lanes by DPP -- and stored
//    into the ring at the slots of the write (codes and scales; v
//    transposed), staged through LDS for whole-row stores.
#include <algorithm>
#include <cmath>

#include "rc_device.h"
#include "rc_kernels.h"

namespace rc {
namespace {

constexpr int kPT = 256;             // tokens per workgroup tile
constexpr int kPN = 128;             // output columns per workgroup tile (one head, d = 128)
constexpr int kPK = 128;             // k bytes per step (two FP8 MFMAs)
constexpr int kPWaves = 8;           // wave w: tokens 32 w .. 32 w + 31, all 128 columns
constexpr int kPThreads = kPWaves * kWave;
constexpr int kABytes = kPT * kPK;   // x tile of a step, 32 KB
constexpr int kBBytes = kPN * kPK;   // W tile of a step, 16 KB
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kDma = kStageBytes / 1024 / kPWaves;  // 1 KB direct-to-LDS loads per wave per step (6)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void glb_void;
typedef __attribute__((address_space(3))) void lds_void;

// 128-byte rows of 8 chunks: chunk c of row r sits at chunk c ^ ((r >> 1) & 7),
// so that the 32 rows a wave reads together spread over the LDS banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int tile_addr(int r, int c) { return r * kPK + ((c ^ swz(r)) << 4); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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
  uint8_t* xq;            // [n_pad][C] workspace
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
  uint8_t* out = a.xq + static_cast<size_t>(t) * a.C;
  for (int c = tid * 8; c < a.C; c += 256 * 8) {
    const v4u w = ok ? *reinterpret_cast<const v4u*>(row + c) : v4u{0u, 0u, 0u, 0u};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = qdiv_rto(__uint_as_float(w[k] << 16), sc, rcp);
      v[2 * k + 1] = qdiv_rto(__uint_as_float(w[k] & 0xFFFF0000u), sc, rcp);
    }
    *reinterpret_cast<uint2*>(out + c) = make_uint2(cvt_fp8x4(v[0], v[1], v[2], v[3]), cvt_fp8x4(v[4], v[5], v[6], v[7]));
  }
  if (tid == 0) a.xs[t] = sc;
}

// Slot of token t of the write (consecutive from head, wrapping from E to A).
__device__ __forceinline__ int write_slot(const ProjArgs& a, int t) {
  const int s = a.head + t;
  return s < a.E ? s : a.r.n_anchor + (s - a.E);
}

__global__ __launch_bounds__(kPThreads) void qkv_proj_kernel(ProjArgs a) {
  // three stages of (x tile, W tile), each its own object: the compiler then
  // sees that reading one stage does not wait for loads into the others
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
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

  // this lane's global source of each of its direct-to-LDS loads: LDS chunk
  // p of a stage (x rows 0..255 then W rows 0..127, 8 chunks a row) holds
  // global chunk (p % 8) ^ swz(row) of its row
  const uint8_t* src[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int p = (wave * kDma + j) * kWave + lane;
    const bool is_x = p < kPT * 8;
    const int r = is_x ? p >> 3 : (p >> 3) - kPT;
    const int c = (p & 7) ^ swz(r);
    src[j] = is_x ? a.xq + static_cast<size_t>(ttok + r) * C + c * 16 : a.w + static_cast<size_t>(col0 + r) * C + c * 16;
  }
  auto issue = [&](uint8_t* st, int s) {  // past the end, the last step is reloaded (nobody reads it)
    const int ss = min(s, S - 1) * kPK;
#pragma unroll
    for (int j = 0; j < kDma; ++j)
      __builtin_amdgcn_global_load_lds((glb_void*)(src[j] + ss), (lds_void*)(st + (wave * kDma + j) * 1024), 16, 0, 0);
  };

  v16f acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = v16f{};
  auto compute = [&](const uint8_t* st) {
    v8i xa[2], wb[4][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      {
        const int r = 32 * wave + n;
        const v4i lo = *reinterpret_cast<const v4i*>(st + tile_addr(r, 4 * ks + 2 * g));
        const v4i hi = *reinterpret_cast<const v4i*>(st + tile_addr(r, 4 * ks + 2 * g + 1));
        xa[ks] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = 32 * b + n;
        const v4i lo = *reinterpret_cast<const v4i*>(st + kABytes + tile_addr(r, 4 * ks + 2 * g));
        const v4i hi = *reinterpret_cast<const v4i*>(st + kABytes + tile_addr(r, 4 * ks + 2 * g + 1));
        wb[b][ks] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[ks], wb[b][ks], acc[b], 0, 0, 0, 0, 0, 0);
  };
  // step s: wait for this thread's loads of step s (those of s + 1 may stay
  // in flight), barrier (all loads of s visible; every wave is done with the
  // stage of s - 1), load step s + 2 into that stage, compute step s
  auto step = [&](uint8_t* cur, uint8_t* free_st, int s) {
    wait_vm<kDma>();
    bare_barrier();
    issue(free_st, s + 2);
    compute(cur);
  };
  issue(st0, 0);
  issue(st1, 1);
  int s = 0;
  for (; s + 3 <= S; s += 3) {
    step(st0, st2, s);
    step(st1, st0, s + 1);
    step(st2, st1, s + 2);
  }
  if (s < S) step(st0, st2, s++);
  if (s < S) step(st1, st0, s++);
  wait_vm<0>();
  __syncthreads();  // all stages free: the epilogue stages through them

  // ---- epilogue.  Accumulator element e of lane (n, g) in column block b
  //      is token tok0 + 8 (e / 4) + 4 g + e % 4, column 32 b + n.
  float swc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) swc[b] = a.w_scale[col0 + 32 * b + n];
  uint8_t* stage = (wave < 6 ? st0 + wave * 8192 : st1 + (wave - 6) * 8192);  // 8 KB per wave
  const size_t hv = static_cast<size_t>(h) * a.r.v_ld;
  {
    const int tok0 = ttok + 32 * wave;
    v16f* ac = acc;
    float sx[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sx[e] = a.xs[tok0 + 8 * (e >> 2) + 4 * g + (e & 3)];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) ac[b][e] *= sx[e] * swc[b];
    if (which == 0) {  // q: bf16, row-major [token][h][128]
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          reinterpret_cast<uint16_t*>(stage)[(8 * (e >> 2) + 4 * g + (e & 3)) * kPN + 32 * b + n] =
              f32_to_bf16(ac[b][e]);
      __builtin_amdgcn_wave_barrier();
      const int r = lane >> 1, half = lane & 1;  // 32 rows x 2 halves of 128 bytes
      const int tok = tok0 + r;
      if (tok < a.n) {
        uint16_t* dst = a.q_out + (static_cast<size_t>(tok) * a.r.H + h) * kPN + 64 * half;
        const uint8_t* sp = stage + r * 256 + 128 * half;
#pragma unroll
        for (int i = 0; i < 8; ++i) reinterpret_cast<v4u*>(dst)[i] = reinterpret_cast<const v4u*>(sp)[i];
      }
      return;
    }
    if (which == 1 && a.use_rope) {  // k: rotate pairs (2j, 2j + 1) = lanes (n, n ^ 1)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const double rev = a.rope.rev[(32 * b + n) >> 1];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = ac[b][e];
          const float xp = __int_as_float(
              __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0xB1, 0xF, 0xF, false));
          float c, sn;
          rope_cs_hw(rev, static_cast<long long>(a.pos0) + tok0 + 8 * (e >> 2) + 4 * g + (e & 3), &c, &sn);
          ac[b][e] = (n & 1) ? fmaf(xp, sn, x * c) : fmaf(-xp, sn, x * c);
        }
      }
    }
    // per (token, head) scale: absmax over the row's 4 values here and 32 lanes
    float sc[16], rc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float m = fmaxf(fmaxf(fabsf(ac[0][e]), fabsf(ac[1][e])), fmaxf(fabsf(ac[2][e]), fabsf(ac[3][e])));
      m = group_max_dpp<16>(m);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      sc[e] = div448(m);
      rc[e] = scale_rcp(sc[e]);
    }
    // codes staged as [token][128] (k) or [128][32 tokens] (v: a column's 32
    // tokens are then one run of bytes)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * g + (e & 3), col = 32 * b + n;
        stage[which == 1 ? r * kPN + col : col * 32 + r] =
            static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(qdiv_rto(ac[b][e], sc[e], rc[e]), 0.f, 0, false));
      }
    __builtin_amdgcn_wave_barrier();
    float* scales = which == 1 ? a.r.k_scale : a.r.v_scale;
    if (n == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = tok0 + 8 * (e >> 2) + 4 * g + (e & 3);
        if (tok < a.n) scales[hv + write_slot(a, tok)] = sc[e];
      }
    }
    if (which == 1) {  // k rows [h][slot][128]
      const int r = lane >> 1, half = lane & 1;
      const int tok = tok0 + r;
      if (tok < a.n) {
        uint8_t* dst = static_cast<uint8_t*>(a.r.k) + (hv + write_slot(a, tok)) * kPN + 64 * half;
        const uint8_t* sp = stage + r * kPN + 64 * half;
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<v4u*>(dst)[i] = reinterpret_cast<const v4u*>(sp)[i];
      }
    } else {  // v transposed [h][col][slot]: lane = (token n, column parity g), so
      // one store instruction writes two runs of 32 consecutive slots (split
      // only where the write wraps)
      const int tok = tok0 + n;
      if (tok < a.n) {
        uint8_t* dst = static_cast<uint8_t*>(a.r.v) + static_cast<size_t>(h) * kPN * a.r.v_ld + write_slot(a, tok);
#pragma unroll 8
        for (int c2 = 0; c2 < kPN / 2; ++c2) {
          const int col = 2 * c2 + g;
          dst[static_cast<size_t>(col) * a.r.v_ld] = stage[col * 32 + n];
        }
      }
    }
    if (which == 2) {
      if (h == 0 && n < 16) {  // slot metadata, once per token: lanes (n < 16, g) take tokens 2n + g
        const int tok = tok0 + 2 * n + g;
        if (tok < a.n) {
          const int sl = write_slot(a, tok);
          a.r.slot_pos[sl] = a.pos0 + tok;
          a.r.slot_block[sl] = a.block_id;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
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
