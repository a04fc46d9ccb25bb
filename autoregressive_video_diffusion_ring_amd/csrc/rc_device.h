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

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16x2 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
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

}  // namespace rc
