// Device-side helpers shared by the RankMixer kernels (gfx950 / CDNA4).
//
// Storage types: `float` (fp32 path) and `bf16_t` (bf16 bit pattern in a uint16_t).
// Every fp32 -> bf16 conversion rounds to nearest, ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmx {

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two bf16 packed in one 32-bit word, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---- 8-element vector access (16 B for bf16, 32 B for fp32); pointers 16 B aligned.
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float* v) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16_t* p, const float* v) {
  uint4 a;
  a.x = pack_bf16x2(v[0], v[1]);
  a.y = pack_bf16x2(v[2], v[3]);
  a.z = pack_bf16x2(v[4], v[5]);
  a.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}

// ---- scalar access
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }

// ---- Token Mixing index map (H = T).  Output row h, column c takes head h of token
// t = c / q at position r = c % q:  M[h, c] = X[t, h*q + r].  Returns the source column
// in token t's row; *t_out receives t.  (RankMixer paper translation, section 3.3.1
// eq (3)-(4); "RankMixer 详解（1）", section 3.1.)  The forward pass and the standalone
// mixing kernel both call this one function.
__device__ __forceinline__ int mix_source(int h, int c, int q, int* t_out) {
  const int t = c / q;
  *t_out = t;
  return h * q + (c - t * q);
}

// ---- wavefront (64 lanes) sum, every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// GELU(u) = u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), the exact (erf) form.
// erf is evaluated with Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (|error| <= 1.5e-7 for all x >= 0, odd extension for x < 0):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),  t = 1 / (1 + p x).
// 1 + erf(x) is formed directly as 2 - q (x >= 0) or q (x < 0), q = poly(t) exp(-x^2), so
// the left tail keeps its relative accuracy.  Branch-free: one reciprocal, one exp2.
__device__ __forceinline__ float gelu_erf(float u) {
  const float x = u * 0.70710678118654752f;
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float q = poly * __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);
  const float one_plus_erf = x >= 0.f ? 2.0f - q : q;
  return 0.5f * u * one_plus_erf;
}

}  // namespace rmx
