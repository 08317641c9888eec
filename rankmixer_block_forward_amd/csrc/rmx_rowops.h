// Row helpers shared by the forward and backward row kernels: W-column chunks (W = 8:
// 16 / 32-byte vectors, W = 1: scalars) of a row held by the 64 lanes of a wavefront,
// chunk c = lane + 64 i at columns c W .. c W + W - 1.
#pragma once

#include "rmx_device.h"

namespace rmx {

template <int W, typename T>
__device__ __forceinline__ void loadw(const T* p, float* v) {
  if constexpr (W == 8) {
    load8(p, v);
  } else {
    v[0] = load1(p);
  }
}
template <int W, typename T>
__device__ __forceinline__ void storew(T* p, const float* v) {
  if constexpr (W == 8) {
    store8(p, v);
  } else {
    store1(p, v[0]);
  }
}

// LayerNorm of one row held as v[NC][W] by the 64 lanes of a wave (chunk c = lane + 64 i),
// in place: v = gamma * (v - mu) / sqrt(var + eps) + beta.
template <int W, int NC, typename T>
__device__ __forceinline__ void wave_layernorm(float (&v)[NC][W], int lane, int nchunks, int D,
                                               const T* gamma, const T* beta, float eps) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
#pragma unroll
      for (int e = 0; e < W; ++e) s += v[i][e];
    }
  }
  const float mu = wave_sum(s) / float(D);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float d = v[i][e] - mu;
        ss += d * d;
      }
    }
  }
  const float var = wave_sum(ss) / float(D);
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float g[W], bt[W];
      loadw<W>(gamma + c * W, g);
      loadw<W>(beta + c * W, bt);
#pragma unroll
      for (int e = 0; e < W; ++e) v[i][e] = g[e] * ((v[i][e] - mu) * rstd) + bt[e];
    }
  }
}


// Backward of the LayerNorm of one row ("RankMixer 详解（1）", section 5.2).  v holds the
// LayerNorm input row, g the gradient its output receives; on return g holds the input
// gradient dr = (q - mean(q) - r_hat mean(q r_hat)) / sqrt(var + eps), q = g gamma,
// r_hat = (v - mu) / sqrt(var + eps), and pg, pb have accumulated the per-column
// gamma and beta gradients g r_hat and g.  The statistics are computed as in
// wave_layernorm.
template <int W, int NC, typename T>
__device__ __forceinline__ void wave_layernorm_backward(const float (&v)[NC][W], float (&g)[NC][W], int lane,
                                                        int nchunks, int D, const T* gamma, float eps,
                                                        float (&pg)[NC][W], float (&pb)[NC][W]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (lane + 64 * i < nchunks)
#pragma unroll
      for (int e = 0; e < W; ++e) s += v[i][e];
  const float mu = wave_sum(s) / float(D);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (lane + 64 * i < nchunks)
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float d = v[i][e] - mu;
        ss += d * d;
      }
  const float var = wave_sum(ss) / float(D);
  const float rstd = 1.0f / sqrtf(var + eps);
  float sq = 0.f, sqr = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) {
      float gm[W];
      loadw<W>(gamma + c * W, gm);
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float rh = (v[i][e] - mu) * rstd;
        pg[i][e] += g[i][e] * rh;
        pb[i][e] += g[i][e];
        g[i][e] *= gm[e];  // q
        sq += g[i][e];
        sqr += g[i][e] * rh;
      }
    }
  }
  const float mq = wave_sum(sq) / float(D), mqr = wave_sum(sqr) / float(D);
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (lane + 64 * i < nchunks)
#pragma unroll
      for (int e = 0; e < W; ++e) g[i][e] = (g[i][e] - mq - (v[i][e] - mu) * rstd * mqr) * rstd;
}

}  // namespace rmx
