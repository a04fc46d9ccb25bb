// Device helpers shared by the ring-cache kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rc {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16x2 (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- fp8 e4m3fn
// gfx950 converts to the OCP e4m3fn format with round-to-nearest-even.
// Values passed here never exceed 448 in magnitude by more than float32
// rounding, which still rounds to 448.
__device__ __forceinline__ uint32_t cvt_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ float fp8_to_f32(uint32_t word, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 3);
  }
}

// ---------------------------------------------------------------- RoPE
// Frequencies theta_j = base^(-2j/d) expressed in revolutions per position
// (theta_j / 2pi), float64, built on the host for each ring.
struct RopeTable {
  double rev[64];
};

// cos and sin of pos * theta_j.  The angle is formed and reduced to
// [-pi, pi] in float64, so positions of a few hundred thousand keep
// float32 accuracy; sincosf then works on a small argument.
__device__ __forceinline__ void rope_cs(const RopeTable& t, int j, long long pos, float* c,
                                        float* s) {
  double r = static_cast<double>(pos) * t.rev[j];
  r -= rint(r);
  float ang = static_cast<float>(r * 6.283185307179586476925286766559);
  sincosf(ang, s, c);
}

// Same, given theta_j / 2pi directly.
__device__ __forceinline__ void rope_cs_rev(double rev, long long pos, float* c, float* s) {
  double r = static_cast<double>(pos) * rev;
  r -= rint(r);
  sincosf(static_cast<float>(r * 6.283185307179586476925286766559), s, c);
}

// cos and sin of pos * theta_j for queries: the angle is reduced in float64
// to at most half a revolution, then the hardware sine and cosine (which take
// revolutions; error about 2^-23 on that range) finish it.  Queries are
// rounded to FP8 or BF16 afterwards (or kept in float32 for the F32 cache,
// whose tolerance is far above this error).
__device__ __forceinline__ void rope_cs_hw(double rev, long long pos, float* c, float* s) {
  double r = static_cast<double>(pos) * rev;
  r -= rint(r);
  const float t = static_cast<float>(r);
  *s = __builtin_amdgcn_sinf(t);
  *c = __builtin_amdgcn_cosf(t);
}

// ---------------------------------------------------------------- masks
// Block-causal visibility of a cached slot (block id kb, -1 = never written)
// to a query of block qb: invisible, visible, or visible with the cache bias
// (the slot belongs to an earlier block).
enum { kVisNone = 0, kVisPlain = 1, kVisBias = 2 };
__device__ __forceinline__ int visibility_class(int kb, int qb) {
  if (kb == -1 || kb > qb) return kVisNone;
  return kb < qb ? kVisBias : kVisPlain;
}

// ---------------------------------------------------------------- reductions
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Maximum over aligned groups of W = 4, 8 or 16 lanes with DPP lane moves
// inside each row of 16 lanes (no LDS round trips): two quad permutes, then
// the half-row mirror (lane i <-> 7 - i) and the row mirror (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_max_dpp(float v) {
  static_assert(W == 4 || W == 8 || W == 16, "DPP group size");
  v = fmaxf(v, dpp_mov<0xB1>(v));  // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_mov<0x4E>(v));  // quad_perm 2,3,0,1
  if constexpr (W >= 8) v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
  if constexpr (W >= 16) v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return v;
}

// a / 448 rounded to nearest (IEEE float32 division) from the reciprocal and
// one FMA correction; checked against the division for every positive float
// whose quotient is a normal number, which holds for a >= 2^-100 (smaller a
// takes the division).
__device__ __forceinline__ float div448(float a) {
  constexpr float y = 1.0f / 448.0f;
  const float q0 = a * y;
  float q = fmaf(fmaf(-q0, 448.0f, a), y, q0);
  if (__ballot(!(a >= 0x1p-100f)) != 0ull) q = a >= 0x1p-100f ? q : a / 448.0f;  // skipped by the wave
  return q;                                                                      // unless a lane needs it
}

// x / scale rounded to float32 with round-to-odd, so that the FP8 conversion
// that follows (round to nearest even) yields the correctly rounded code of
// the exact quotient.  A plain float32 quotient can land exactly on a
// midpoint between two FP8 codes when the exact quotient lies just beside it
// (common for unrotated input: x and the absmax carry 8 significant bits, so
// 448 x / absmax is often a short fraction, while scale = absmax / 448 is
// rounded), and the conversion's tie-break would then round the wrong way.
// Round-to-odd keeps the "inexact" information in the last bit (float32 has
// 20 more bits than e4m3), the classical remedy for double rounding.
//
// The quotient comes from rcp ~ 1/scale and one Newton step, which leaves it
// within one ulp of x / scale; the remainder x - q scale is then exact (one
// FMA), and its sign gives the truncation and the sticky bit.  Callers pass
// rcp = 0 for an all-zero row (scale 0), which yields 0.
__device__ __forceinline__ float qdiv_rto(float x, float scale, float rcp) {
  const float q0 = x * rcp;
  const float e0 = fmaf(-q0, scale, x);
  const float q = fmaf(e0, rcp, q0);
  const float e = fmaf(-q, scale, x);
  const uint32_t u = __float_as_uint(q);
  const uint32_t t = (u - ((__float_as_uint(e) ^ u) >> 31)) | 1u;  // toward zero if e opposes q
  return e == 0.f ? q : __uint_as_float(t);
}

// Reciprocal of a row scale for the quotients above (0 for a zero row).
__device__ __forceinline__ float scale_rcp(float scale) {
  return scale > 0.f ? __builtin_amdgcn_rcpf(scale) : 0.f;
}

}  // namespace rc
