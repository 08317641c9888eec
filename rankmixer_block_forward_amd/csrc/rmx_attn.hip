// Self-attention routing: the comparator of the pages' routing ablation ("RankMixer" paper
// translation, section 4.4; written out as single-head attention in "RankMixer 详解（1）",
// section 3.4): in place of Token Mixing, every token of a sample attends to all T tokens,
//   A = softmax(Q K^T / sqrt(D)) V,  Q = X Wq, K = X Wk, V = X Wv,
// and the block continues with S = LN1(A + X).  Q, K, V come from the grouped-GEMM kernels
// (one product each over the B*T rows); this kernel does the scores, the softmax, the
// weighted sum, the residual and LN1 for one sample per workgroup.
//
// Each wave owns QG query rows at a time (held in registers), streams the sample's T key
// rows to form the QG x T scores (wave-wide dot products), keeps score j in lane j for the
// softmax (T <= 64), then streams the T value rows and sums them with the probabilities,
// which lanes broadcast with readlane.  Everything is fp32; Q, K, V, X are read in the
// storage type and S is written token-major [T, B, D] for the per-token FFN.
#include "rmx_device.h"
#include "rmx_internal.h"
#include "rmx_rowops.h"

namespace rmx {

namespace {

constexpr int ATTN_MAX_WAVES = 8;

template <typename T, int W, int NC, int QG>
__global__ __launch_bounds__(64 * ATTN_MAX_WAVES) void attn_rows_kernel(AttnArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int Tn = a.T, D = a.D, B = a.B;
  const int nchunks = D / W;
  const float scale = 1.0f / sqrtf(float(D));
  const size_t base = size_t(b) * Tn * D;
  const T* Q = static_cast<const T*>(a.Q) + base;
  const T* K = static_cast<const T*>(a.K) + base;
  const T* V = static_cast<const T*>(a.V) + base;
  const T* X = static_cast<const T*>(a.X) + base;

  auto load_row = [&](const T* src, float (&v)[NC][W]) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) {
        loadw<W>(src + c * W, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) v[i][e] = 0.f;
      }
    }
  };

  for (int t0 = wave * QG; t0 < Tn; t0 += nw * QG) {
    float q[QG][NC][W];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (t0 + g < Tn) {
        load_row(Q + size_t(t0 + g) * D, q[g]);
      } else {
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
          for (int e = 0; e < W; ++e) q[g][i][e] = 0.f;
      }
    }
    // scores: lane j keeps q_g . k_j / sqrt(D)
    float sc[QG];
#pragma unroll
    for (int g = 0; g < QG; ++g) sc[g] = -INFINITY;
    for (int j = 0; j < Tn; ++j) {
      float k[NC][W];
      load_row(K + size_t(j) * D, k);
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
          for (int e = 0; e < W; ++e) s = fmaf(q[g][i][e], k[i][e], s);
        s = wave_sum(s);
        if (lane == j) sc[g] = s * scale;
      }
    }
    // softmax along the keys (lanes j < T)
    float p[QG];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      const float m = wave_max(sc[g]);
      const float ex = lane < Tn ? __expf(sc[g] - m) : 0.f;
      p[g] = ex / wave_sum(ex);
    }
    // weighted sum of the value rows
    float acc[QG][NC][W];
#pragma unroll
    for (int g = 0; g < QG; ++g)
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int e = 0; e < W; ++e) acc[g][i][e] = 0.f;
    for (int j = 0; j < Tn; ++j) {
      float v[NC][W];
      load_row(V + size_t(j) * D, v);
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[g]), j));
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
          for (int e = 0; e < W; ++e) acc[g][i][e] = fmaf(pj, v[i][e], acc[g][i][e]);
      }
    }
    // residual and LN1, written token-major
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      const int t = t0 + g;
      if (t >= Tn) break;
      float x[NC][W];
      load_row(X + size_t(t) * D, x);
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int e = 0; e < W; ++e) acc[g][i][e] += x[i][e];
      wave_layernorm<W, NC>(acc[g], lane, nchunks, D, static_cast<const T*>(a.ln1_g), static_cast<const T*>(a.ln1_b),
                            a.eps);
      T* dst = static_cast<T*>(a.S) + (size_t(t) * B + b) * D;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunks) storew<W>(dst + c * W, acc[g][i]);
      }
    }
  }
}

template <typename T, int W, int NC, int QG>
hipError_t launch_nc(const AttnArgs& a, hipStream_t stream) {
  const int groups = (a.T + QG - 1) / QG;
  const int nw = groups < ATTN_MAX_WAVES ? groups : ATTN_MAX_WAVES;
  hipLaunchKernelGGL((attn_rows_kernel<T, W, NC, QG>), dim3(a.B), dim3(64 * nw), 0, stream, a);
  return hipGetLastError();
}

// query rows per wave pass: as many as the registers of a row allow
template <typename T>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  if (!rows_vectorized(a.T, a.D)) return launch_nc<T, 1, ROWS_MAX_D_SCALAR / 64, 2>(a, stream);
  switch ((a.D / 8 + 63) / 64) {
    case 1: return launch_nc<T, 8, 1, 4>(a, stream);
    case 2: return launch_nc<T, 8, 2, 4>(a, stream);
    case 3: return launch_nc<T, 8, 3, 2>(a, stream);
    default: return launch_nc<T, 8, 4, 1>(a, stream);
  }
}

}  // namespace

bool attn_supported(int dtype, int T, int D) {
  (void)dtype;
  if (T > ATTN_MAX_T || D % T) return false;
  return rows_vectorized(T, D) ? D <= ATTN_MAX_D : D <= ROWS_MAX_D_SCALAR;
}

hipError_t launch_attn_rows(int dtype, const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_t<bf16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace rmx
