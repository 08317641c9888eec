// Row passes of the block backward, and the batch sums of the bias / LayerNorm gradients.
//
// Gradients as "RankMixer 详解（1）：特征分组与完整计算流程" section 5.2 writes them for one
// sample: the mean pool sends g_o / T to every row of X_L; LayerNorm backward
// dr = (q - mean(q) - r_hat mean(q r_hat)) / sqrt(var + eps) with q = g gamma; Token Mixing
// sends its output gradient back through P^T, and with the first residual the block input
// receives (P^T + I) g.  P is a symmetric permutation, so P^T g is read through the same
// index map (mix_source) as the forward mixing.
//
// One workgroup per sample b.  Modes:
//   BWD_TOP     block L: gY = LN2_backward(g_o / T) from the saved pre-LN2 rows Y_L.
//   BWD_MID     between block n (n >= 2) and block n - 1: recompute X_{n-1} = LN2(Y_{n-1})
//               into LDS exactly as the forward row kernel does (rounded to the storage
//               type), form R1 = mix(X_{n-1}) + X_{n-1} row by row, gR = LN1_backward(gS),
//               write gR to a per-sample scratch, then gX = gR + P^T gR and
//               gY_{n-1} = LN2_backward(gX) from Y_{n-1}.
//   BWD_BOTTOM  block 1: as BWD_MID with X_0 itself in LDS, ending with dX = gR + P^T gR.
// Per-sample partial sums of the LayerNorm parameter gradients (over the T rows, in wave
// order) go to [B, D] buffers; colsum_kernel then sums over samples in a fixed order.
#include "rmx_device.h"
#include "rmx_internal.h"
#include "rmx_rowops.h"

namespace rmx {

namespace {

constexpr int BWD_MAX_WAVES = 8;

// Per-wave partial sums meet in LDS (red: [nw][D] fp32), summed over waves in wave order.
template <int W, int NC>
__device__ __forceinline__ void reduce_partials(float* red, const float (&pg)[NC][W], const float (&pb)[NC][W],
                                                float* out_g, float* out_b, int lane, int wave, int nw,
                                                int nchunks, int D) {
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks)
#pragma unroll
        for (int e = 0; e < W; ++e) red[wave * D + c * W + e] = half ? pb[i][e] : pg[i][e];
    }
    __syncthreads();
    float* out = half ? out_b : out_g;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[w * D + d];
      out[d] = s;
    }
    __syncthreads();
  }
}

template <typename T, int W, int NC, int MODE>
__global__ __launch_bounds__(64 * BWD_MAX_WAVES) void rows_bwd_kernel(RowsBwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int Tn = a.T, D = a.D, B = a.B;
  const int q = D / Tn;
  const int nchunks = D / W;
  T* xs = reinterpret_cast<T*>(smem_raw);          // [T][D] block input rows of sample b
  float* red = reinterpret_cast<float*>(smem_raw);  // [nw][D], reused once xs is consumed
  float* gR = a.gR + size_t(b) * Tn * D;            // [T][D] scratch of sample b

  float pg[NC][W], pb[NC][W];
  auto zero_partials = [&]() {
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < W; ++e) pg[i][e] = pb[i][e] = 0.f;
  };
  // LN2 backward of pre-LN2 row Y[t, b] with upstream gradient g; writes gY (fp32 and the
  // storage type, both token-major [T, B, D]).
  auto ln2_backward_row = [&](const float* Y, const T* gamma, int t, float (&g)[NC][W]) {
    float y[NC][W];
    const float* src = Y + (size_t(t) * B + b) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane + 64 * i < nchunks) loadw<W>(src + (lane + 64 * i) * W, y[i]);
    wave_layernorm_backward<W, NC>(y, g, lane, nchunks, D, gamma, a.eps, pg, pb);
    float* d32 = a.gY32 + (size_t(t) * B + b) * D;
    T* dlo = static_cast<T*>(a.gY) + (size_t(t) * B + b) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) {
        storew<W>(d32 + c * W, g[i]);
        storew<W>(dlo + c * W, g[i]);
      }
    }
  };

  if constexpr (MODE == BWD_TOP) {
    zero_partials();
    for (int t = wave; t < Tn; t += nw) {
      float g[NC][W];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunks) {
          loadw<W>(a.g_out + size_t(b) * D + c * W, g[i]);
#pragma unroll
          for (int e = 0; e < W; ++e) g[i][e] /= float(Tn);
        }
      }
      ln2_backward_row(a.Y, static_cast<const T*>(a.ln2_g), t, g);
    }
    reduce_partials<W, NC>(red, pg, pb, a.part_ln2 + size_t(b) * D, a.part_ln2 + (size_t(B) + b) * D, lane, wave,
                           nw, nchunks, D);
    return;
  }

  // Phase 1: the block input rows into LDS.
  for (int t = wave; t < Tn; t += nw) {
    float v[NC][W];
    if constexpr (MODE == BWD_BOTTOM) {
      const T* src = static_cast<const T*>(a.X0) + (size_t(b) * Tn + t) * D;
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (lane + 64 * i < nchunks) loadw<W>(src + (lane + 64 * i) * W, v[i]);
    } else {
      const float* src = a.Y + (size_t(t) * B + b) * D;
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (lane + 64 * i < nchunks) loadw<W>(src + (lane + 64 * i) * W, v[i]);
      wave_layernorm<W, NC>(v, lane, nchunks, D, static_cast<const T*>(a.ln2_g), static_cast<const T*>(a.ln2_b),
                            a.eps);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) storew<W>(xs + t * D + c * W, v[i]);
    }
  }
  __syncthreads();

  // Phase 2: gR[h] = LN1_backward(gS[h]) with R1[h] = X[h] + mix(X)[h].
  zero_partials();
  for (int h = wave; h < Tn; h += nw) {
    float r[NC][W], g[NC][W];
    const float* gs = a.gS + (size_t(h) * B + b) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) {
        const int col = c * W;
        int t;
        const int sc = mix_source(h, col, q, &t);  // W consecutive columns stay in one head
        float own[W], mixed[W];
        loadw<W>(xs + h * D + col, own);
        loadw<W>(xs + t * D + sc, mixed);
#pragma unroll
        for (int e = 0; e < W; ++e) r[i][e] = own[e] + mixed[e];
        loadw<W>(gs + col, g[i]);
      }
    }
    wave_layernorm_backward<W, NC>(r, g, lane, nchunks, D, static_cast<const T*>(a.ln1_g), a.eps, pg, pb);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) storew<W>(gR + h * D + c * W, g[i]);
    }
  }
  // the barrier publishes gR to the workgroup (global memory, workgroup scope) and frees xs
  __syncthreads();
  reduce_partials<W, NC>(red, pg, pb, a.part_ln1 + size_t(b) * D, a.part_ln1 + (size_t(B) + b) * D, lane, wave, nw,
                         nchunks, D);

  // Phase 3: gX[t] = gR[t] + (P^T gR)[t], then dX (block 1) or LN2 backward of block n - 1.
  zero_partials();
  for (int t = wave; t < Tn; t += nw) {
    float g[NC][W];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) {
        const int col = c * W;
        int h;
        const int sc = mix_source(t, col, q, &h);
        float own[W], back[W];
        loadw<W>(gR + t * D + col, own);
        loadw<W>(gR + h * D + sc, back);
#pragma unroll
        for (int e = 0; e < W; ++e) g[i][e] = own[e] + back[e];
      }
    }
    if constexpr (MODE == BWD_BOTTOM) {
      float* dst = a.dX + (size_t(b) * Tn + t) * D;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunks) storew<W>(dst + c * W, g[i]);
      }
    } else {
      ln2_backward_row(a.Y, static_cast<const T*>(a.ln2_g), t, g);
    }
  }
  if constexpr (MODE == BWD_MID)
    reduce_partials<W, NC>(red, pg, pb, a.part_ln2 + size_t(b) * D, a.part_ln2 + (size_t(B) + b) * D, lane, wave,
                           nw, nchunks, D);
}

// out[g, rs, n] = sum of rows rs * rows_per .. of in[g, :, n] (fixed row order per lane,
// then the waves in order).  W columns per lane.
template <typename T, int W>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ in, float* __restrict__ out, int R,
                                                     int N, int rows_per) {
  __shared__ float red[4][64 * W];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.y, rs = blockIdx.z, RS = gridDim.z;
  const int col = (blockIdx.x * 64 + lane) * W;
  const int r0 = rs * rows_per, r1 = min(R, r0 + rows_per);
  float acc[W];
#pragma unroll
  for (int e = 0; e < W; ++e) acc[e] = 0.f;
  if (col < N) {
    const T* src = in + size_t(g) * R * N + col;
#pragma unroll 4
    for (int r = r0 + wave; r < r1; r += 4) {
      float v[W];
      loadw<W>(src + size_t(r) * N, v);
#pragma unroll
      for (int e = 0; e < W; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < W; ++e) red[wave][lane * W + e] = acc[e];
  __syncthreads();
  if (wave == 0 && col < N) {
    float s[W];
#pragma unroll
    for (int e = 0; e < W; ++e) s[e] = red[0][lane * W + e] + red[1][lane * W + e] + red[2][lane * W + e] +
                                      red[3][lane * W + e];
    float* dst = out + (size_t(g) * RS + rs) * N + col;
#pragma unroll
    for (int e = 0; e < W; ++e) dst[e] = s[e];
  }
}

template <typename T, int W, int NC>
hipError_t launch_rows_bwd_nc(int mode, const RowsBwdArgs& a, hipStream_t stream) {
  const int nw = a.T < BWD_MAX_WAVES ? a.T : BWD_MAX_WAVES;
  const size_t lds = rows_bwd_lds_bytes(sizeof(T) == 2 ? DT_BF16 : DT_FP32, a.T, a.D);
  const dim3 grid(a.B), block(64 * nw);
  switch (mode) {
    case BWD_TOP: hipLaunchKernelGGL((rows_bwd_kernel<T, W, NC, BWD_TOP>), grid, block, lds, stream, a); break;
    case BWD_MID: hipLaunchKernelGGL((rows_bwd_kernel<T, W, NC, BWD_MID>), grid, block, lds, stream, a); break;
    default: hipLaunchKernelGGL((rows_bwd_kernel<T, W, NC, BWD_BOTTOM>), grid, block, lds, stream, a); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rows_bwd_t(int mode, const RowsBwdArgs& a, hipStream_t stream) {
  if (!rows_vectorized(a.T, a.D)) return launch_rows_bwd_nc<T, 1, ROWS_BWD_MAX_D_SCALAR / 64>(mode, a, stream);
  switch ((a.D / 8 + 63) / 64) {
    case 1: return launch_rows_bwd_nc<T, 8, 1>(mode, a, stream);
    case 2: return launch_rows_bwd_nc<T, 8, 2>(mode, a, stream);
    case 3: return launch_rows_bwd_nc<T, 8, 3>(mode, a, stream);
    default: return launch_rows_bwd_nc<T, 8, 4>(mode, a, stream);
  }
}

template <typename T, int W, int NC>
hipError_t set_lds_limit_nc() {
  const int bytes = int(ROWS_BWD_MAX_LDS);
  hipError_t e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_bwd_kernel<T, W, NC, BWD_TOP>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_bwd_kernel<T, W, NC, BWD_MID>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess)
    return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_bwd_kernel<T, W, NC, BWD_BOTTOM>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename T>
hipError_t set_lds_limit() {
  hipError_t e;
  if ((e = set_lds_limit_nc<T, 1, ROWS_BWD_MAX_D_SCALAR / 64>()) != hipSuccess) return e;
  if ((e = set_lds_limit_nc<T, 8, 1>()) != hipSuccess) return e;
  if ((e = set_lds_limit_nc<T, 8, 2>()) != hipSuccess) return e;
  if ((e = set_lds_limit_nc<T, 8, 3>()) != hipSuccess) return e;
  return set_lds_limit_nc<T, 8, 4>();
}

template <typename T, int W>
hipError_t launch_colsum_w(const T* in, float* out, float* scratch, int G, int R, int N, hipStream_t stream) {
  // rows split over up to COLSUM_MAX_SPLIT workgroups per column block, then the partial
  // sums [G][RS][N] summed by a second pass
  const int cols = (N / W + 63) / 64;
  int RS = (R + COLSUM_ROWS - 1) / COLSUM_ROWS;
  if (RS > COLSUM_MAX_SPLIT) RS = COLSUM_MAX_SPLIT;
  if (RS <= 1) {
    hipLaunchKernelGGL((colsum_kernel<T, W>), dim3(cols, G, 1), dim3(256), 0, stream, in, out, R, N, R);
    return hipGetLastError();
  }
  const int rows_per = (R + RS - 1) / RS;
  hipLaunchKernelGGL((colsum_kernel<T, W>), dim3(cols, G, RS), dim3(256), 0, stream, in, scratch, R, N, rows_per);
  hipLaunchKernelGGL((colsum_kernel<float, W>), dim3(cols, G, 1), dim3(256), 0, stream,
                     static_cast<const float*>(scratch), out, RS, N, RS);
  return hipGetLastError();
}

}  // namespace

bool rows_bwd_supported(int dtype, int T, int D) {
  if (D % T) return false;
  const size_t lds = rows_bwd_lds_bytes(dtype, T, D);
  if (lds > ROWS_BWD_MAX_LDS) return false;
  return rows_vectorized(T, D) ? D <= ROWS_BWD_MAX_D : D <= ROWS_BWD_MAX_D_SCALAR;
}

size_t rows_bwd_lds_bytes(int dtype, int T, int D) {
  const int nw = T < BWD_MAX_WAVES ? T : BWD_MAX_WAVES;
  const size_t xs = size_t(T) * D * dtype_size(dtype), red = size_t(nw) * D * 4;
  return xs > red ? xs : red;
}

hipError_t rows_bwd_init() {
  hipError_t e = set_lds_limit<float>();
  if (e != hipSuccess) return e;
  return set_lds_limit<bf16_t>();
}

hipError_t launch_rows_bwd(int dtype, int mode, const RowsBwdArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  return dtype == DT_BF16 ? launch_rows_bwd_t<bf16_t>(mode, a, stream) : launch_rows_bwd_t<float>(mode, a, stream);
}

hipError_t launch_colsum(int dtype, const void* in, float* out, float* scratch, int G, int R, int N,
                         hipStream_t stream) {
  if (G == 0 || N == 0 || R == 0) return hipSuccess;
  const bool vec = N % 8 == 0;
  if (dtype == DT_BF16) {
    const bf16_t* p = static_cast<const bf16_t*>(in);
    return vec ? launch_colsum_w<bf16_t, 8>(p, out, scratch, G, R, N, stream)
               : launch_colsum_w<bf16_t, 1>(p, out, scratch, G, R, N, stream);
  }
  const float* p = static_cast<const float*>(in);
  return vec ? launch_colsum_w<float, 8>(p, out, scratch, G, R, N, stream)
             : launch_colsum_w<float, 1>(p, out, scratch, G, R, N, stream);
}

}  // namespace rmx
