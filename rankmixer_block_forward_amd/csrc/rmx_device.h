// Device-side helpers shared by the RankMixer kernels (gfx950 / CDNA4).
//
// Storage types: `float` (fp32 path) and `bf16_t` (bf16 bit pattern in a uint16_t).
// Every fp32 -> bf16 conversion rounds to nearest, ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmx_layout.h"

namespace rmx {

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even; NaN stays NaN.  gfx950 converts in one instruction
// (v_cvt_pk_bf16_f32, two values at a time).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two bf16 packed in one 32-bit word, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return uint16_t(pack_bf16x2(f, 0.f)); }

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

// The packed bf16 and MXFP8 operand layouts (pk_off, mx_off, mx_scale_off, ...) are in
// rmx_layout.h.

// Biased E8M0 scale of a block whose largest magnitude is amax: 2^(floor(log2 amax) - 8),
// 8 the top exponent of E4M3, clamped below at 2^-127 (an all-zero block takes 2^-127).
// From the fp32 exponent field e: floor(log2 amax) - 8 + 127 = e - 8.
__device__ __forceinline__ uint32_t mx_scale_bits(float amax) {
  const uint32_t e = (__float_as_uint(amax) >> 23) & 0xffu;
  return e > 8u ? e - 8u : 0u;
}
// 1 / scale as fp32: 2^(127 - bits), a normal number for every bits the above returns.
__device__ __forceinline__ float mx_inv_scale(uint32_t bits) { return __uint_as_float((254u - bits) << 23); }
// Eight values (already multiplied by 1 / scale) to E4M3 codes, round to nearest even,
// saturating at +-448 (the conversion itself would give NaN from 480 up); byte e = v[e].
__device__ __forceinline__ uint2 e4m3_pack8(const float* v) {
  auto sat = [](float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); };
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v[0]), sat(v[1]), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v[2]), sat(v[3]), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v[4]), sat(v[5]), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v[6]), sat(v[7]), hi, true);
  return make_uint2(lo, hi);
}

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

// ---- cross-lane exchanges through DPP (the VALU reads a neighbouring lane directly), not
// through LDS-routed shuffles.  dpp_take<CTRL>(v) returns v of the lane that the DPP control
// CTRL names: 0xB1 = quad_perm [1,0,3,2] (lane ^ 1), 0x4E = quad_perm [2,3,0,1] (lane ^ 2),
// 0x141 = row_half_mirror (lane i <-> 7 - i within 8), 0x140 = row_mirror (i <-> 15 - i
// within 16).  Callers run them with every lane of the wave active; a lane read while
// inactive would give the `old` operand 0.
template <int CTRL>
__device__ __forceinline__ float dpp_take(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Maximum over the 4 lanes of a quad (lanes 4i .. 4i + 3, the lanes that hold one MX scale
// block); every lane of the quad receives it.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_take<0xB1>(v));
  return fmaxf(v, dpp_take<0x4E>(v));
}

// Wavefront (64 lanes) sum; every lane receives the same total.  Butterflies within each
// 16-lane row (each pairwise sum is formed by both partners, so the lanes of a row agree bit
// for bit), then the four row sums read from lanes 0, 16, 32, 48 and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_take<0xB1>(v);
  v += dpp_take<0x4E>(v);
  v += dpp_take<0x141>(v);
  v += dpp_take<0x140>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Wavefront maximum, the same pattern.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_take<0xB1>(v));
  v = fmaxf(v, dpp_take<0x4E>(v));
  v = fmaxf(v, dpp_take<0x141>(v));
  v = fmaxf(v, dpp_take<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// GELU(u) = u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), the exact (erf) form.
// erf is evaluated with Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (|error| <= 1.5e-7 for all x >= 0, odd extension for x < 0):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),  t = 1 / (1 + p x).
// With x = |u| / sqrt 2 and q = (1 - erf(x)) / 2 (the a_k halved), Phi(u) = 1 - q for
// u >= 0 and q for u < 0, so the left tail keeps its relative accuracy.  The 1 / sqrt 2
// is folded into p and into the exponent: exp(-x^2) = exp2(-u^2 log2(e) / 2).
// The pieces shared by the two GELU entry points below: for a = |u|,
// t = 1 / (1 + p a / sqrt 2), poly = (a1 + a2 t + ... + a5 t^4) / 2 and e = exp(-u^2 / 2),
// so that q = (1 - erf(a / sqrt 2)) / 2 = t poly e.
struct NormalTail {
  float a, t, poly, e;
};
__device__ __forceinline__ NormalTail normal_tail(float u) {
  NormalTail r;
  r.a = fabsf(u);
  r.t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, r.a, 1.0f));
  float poly = fmaf(0.5307027145f, r.t, -0.7265760135f);
  poly = fmaf(poly, r.t, 0.7107068705f);
  poly = fmaf(poly, r.t, -0.142248368f);
  r.poly = fmaf(poly, r.t, 0.127414796f);
  r.e = __builtin_amdgcn_exp2f((u * -0.72134752044448170f) * u);
  return r;
}

// GELU in the form u Phi(u) = max(u, 0) - |u| q (u q for u < 0, u (1 - q) for u >= 0), with
// |u| q grouped as (|u| t)(poly e) so that the last step is one fused multiply-add:
// 11 VALU operations (6 fused multiply-adds, 4 multiplies, a max), one reciprocal, one
// exp2, branch-free.
__device__ __forceinline__ float gelu_from_tail(float u, const NormalTail& n) {
  return fmaf(-(n.a * n.t), n.poly * n.e, fmaxf(u, 0.0f));
}

__device__ __forceinline__ float gelu_erf(float u) { return gelu_from_tail(u, normal_tail(u)); }

// GELU(u) and its derivative GELU'(u) = Phi(u) + u phi(u), phi(u) = exp(-u^2 / 2) /
// sqrt(2 pi) the standard normal density ("RankMixer 详解（1）", section 5.2), from one erf
// evaluation: the exponential of the tail serves phi as well.  The value is computed
// exactly as gelu_erf computes it.
__device__ __forceinline__ float gelu_erf_and_grad(float u, float* grad) {
  const NormalTail n = normal_tail(u);
  const float q = n.t * (n.poly * n.e);
  const float Phi = u >= 0.f ? 1.0f - q : q;
  *grad = fmaf(u * 0.39894228040143268f, n.e, Phi);
  return gelu_from_tail(u, n);
}

}  // namespace rmx
