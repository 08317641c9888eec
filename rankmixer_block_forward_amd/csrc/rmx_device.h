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

// Exact GELU, u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), erf from the device math library.
__device__ __forceinline__ float gelu_exact(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

}  // namespace rmx
