// Row kernel of the RankMixer block: everything between two grouped GEMMs.
//
// One workgroup owns one sample b (its T x D token matrix).  Depending on the mode it
//   - reads the previous block's pre-LN2 rows Y[t, b, :] (fp32) and applies LN2, or
//     reads the input X0[b, t, :] as is (first block);
//   - keeps the resulting X[b] in LDS, then for every output row h forms
//     R[h, c] = X[h, c] + X[t, h*q + r] (c = t*q + r: Token Mixing with H = T folded into
//     the LDS read address, residual added on the fly) and applies LN1, writing
//     S[h, b, :] token-major for the grouped GEMMs;
//   - or, after the last block, mean-pools the LN2 output over tokens.
// RankMixer paper translation, section 3.1 eq (1), 3.3.1 eq (3)-(5);
// "RankMixer 详解（1）", sections 3.1 (index map), 3.3 (LayerNorm), 5.1 (pool).
//
// LayerNorm statistics are two-pass (mean, then mean of squared deviations) in fp32
// over values held in registers, reduced across the 64 lanes of one wavefront.
#include <type_traits>

#include "rmx_device.h"
#include "rmx_internal.h"
#include "rmx_rowops.h"

namespace rmx {

namespace {

// One block input row (token t of sample b) into registers: X0[b, t] (first block) or the
// previous block's pre-LN2 row Y[t, b] (fp32), which after a Sparse-MoE block is the
// combine S[t, b] + sum over its active experts e, in expert order, of the gate-scaled
// expert row (RankMixer paper translation, section 3.4 eq (10), plus the block residual).
template <typename T, int W, int NC, int MODE, bool MOE>
__device__ __forceinline__ void load_row(const RowsArgs& a, int b, int t, int lane, int nchunks,
                                         float (&v)[NC][W]) {
  if constexpr (MOE) {
    const T* src = static_cast<const T*>(a.in) + (size_t(t) * a.B + b) * a.D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) loadw<W>(src + c * W, v[i]);
    }
    // The expert rows BAT at a time: a batch's row indices (wave-uniform scalars), then
    // every load of the batch in flight, held as raw bf16 until added.  An inactive
    // expert's load reads the S row again (cached) and its add is skipped, so the sum
    // runs over the active experts in expert order.
    const int* pos = a.moe_pos + size_t(t) * a.moe_E * a.B + b;
    const int E = a.moe_E;
    // registers of one expert row: NC x 4 (W = 8, 8 bf16 in 16 bytes) or NC (W = 1)
    constexpr int PER = W == 8 ? NC * 4 : NC, BAT0 = 36 / PER;
    constexpr int BAT = BAT0 < 1 ? 1 : (BAT0 > 4 ? 4 : BAT0);
    using Raw = typename std::conditional<W == 8, uint4, uint16_t>::type;
#pragma unroll 1
    for (int e0 = 0; e0 < E; e0 += BAT) {
      int r[BAT];
#pragma unroll
      for (int j = 0; j < BAT; ++j) r[j] = e0 + j < E ? pos[size_t(e0 + j) * a.B] : -1;
      Raw u[BAT][NC];
#pragma unroll
      for (int j = 0; j < BAT; ++j) {
        const T* ye = r[j] >= 0 ? static_cast<const T*>(a.moe_ye) + size_t(r[j]) * a.D : src;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int c = lane + 64 * i;
          if (c < nchunks) u[j][i] = *reinterpret_cast<const Raw*>(ye + c * W);
        }
      }
#pragma unroll
      for (int j = 0; j < BAT; ++j) {
        if (r[j] >= 0) {
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            if (c < nchunks) {
              if constexpr (W == 8) {
                const uint32_t wd[4] = {u[j][i].x, u[j][i].y, u[j][i].z, u[j][i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  v[i][2 * k] += __uint_as_float(wd[k] << 16);
                  v[i][2 * k + 1] += __uint_as_float(wd[k] & 0xffff0000u);
                }
              } else {
                v[i][0] += bf16_to_f32(u[j][i]);
              }
            }
          }
        }
      }
    }
    return;
  }
  if constexpr (MODE == ROWS_FIRST) {
    const T* src = static_cast<const T*>(a.in) + (size_t(b) * a.T + t) * a.D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) loadw<W>(src + c * W, v[i]);
    }
  } else {
    const float* src = static_cast<const float*>(a.in) + (size_t(t) * a.B + b) * a.D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) loadw<W>(src + c * W, v[i]);
    }
  }
}

// NC = chunks of W columns per lane (ceil(D / (64 W))).  Up to rows_max_waves waves per
// sample; each
// wave walks its tokens with the next row's loads in flight while the current one is
// normalized.
// Waves per sample: 16, or 8 where the registers of a wide row (or the pool's partial sums)
// need the room.
constexpr int rows_max_waves(int NC, int MODE, bool MOE = false) {
  return MODE == ROWS_FINAL ? (NC > 4 ? 4 : 8) : (NC > 3 ? 8 : 16);
}

template <typename T, int W, int NC, int MODE, bool MOE = false>
__global__ __launch_bounds__(64 * rows_max_waves(NC, MODE, MOE)) void rows_kernel(RowsArgs a) {
  static_assert(!MOE || (MODE != ROWS_FIRST && sizeof(T) == 2), "the combine follows a bf16 Sparse-MoE block");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int Tn = a.T, D = a.D, B = a.B;
  const int q = D / Tn;
  const int nchunks = D / W;
  T* xs = reinterpret_cast<T*>(smem_raw);  // [T][D] rows of sample b (FIRST / MID)

  float pacc[MODE == ROWS_FINAL ? NC : 1][W];
#pragma unroll
  for (int i = 0; i < (MODE == ROWS_FINAL ? NC : 1); ++i)
#pragma unroll
    for (int e = 0; e < W; ++e) pacc[i][e] = 0.f;

  // Phase A: the block input rows X[b, t, :] for t = wave, wave + nw, ...
  float nxt[NC][W];
  if (wave < Tn) load_row<T, W, NC, MODE, MOE>(a, b, wave, lane, nchunks, nxt);
  for (int t = wave; t < Tn; t += nw) {
    float v[NC][W];
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < W; ++e) v[i][e] = nxt[i][e];
    if (t + nw < Tn) load_row<T, W, NC, MODE, MOE>(a, b, t + nw, lane, nchunks, nxt);
    if constexpr (MODE == ROWS_FIRST) {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunks) storew<W>(xs + t * D + c * W, v[i]);
      }
    } else {
      wave_layernorm<W, NC>(v, lane, nchunks, D, static_cast<const T*>(a.ln2_g),
                            static_cast<const T*>(a.ln2_b), a.eps);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunks) {
          if constexpr (MODE == ROWS_MID) {
            storew<W>(xs + t * D + c * W, v[i]);
          } else {
#pragma unroll
            for (int e = 0; e < W; ++e) pacc[i][e] += v[i][e];
            if (a.xl) storew<W>(static_cast<T*>(a.xl) + (size_t(b) * Tn + t) * D + c * W, v[i]);
          }
        }
      }
    }
  }

  if constexpr (MODE == ROWS_FINAL) {
    // Mean pool: per-wave partial sums meet in LDS, then sum over waves in wave order.
    float* red = reinterpret_cast<float*>(smem_raw);  // [nw][D]
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks)
#pragma unroll
        for (int e = 0; e < W; ++e) red[wave * D + c * W + e] = pacc[i][e];
    }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[w * D + d];
      a.pool[size_t(b) * D + d] = s / float(Tn);
    }
    return;
  }

  __syncthreads();
  // Phase B: output rows h = wave, wave + nw, ...:  S[h] = LN1(X[h] + mix(X)[h]).
  for (int h = wave; h < Tn; h += nw) {
    float r[NC][W];
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
      }
    }
    wave_layernorm<W, NC>(r, lane, nchunks, D, static_cast<const T*>(a.ln1_g),
                          static_cast<const T*>(a.ln1_b), a.eps);
    if constexpr (W == 8) {
      if (a.s_packed) {
        T* dst = static_cast<T*>(a.S) + size_t(h) * size_t(pk_rows(B)) * D;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int c = lane + 64 * i;
          if (c < nchunks) storew<W>(dst + pk_off(b, c * W, D), r[i]);
        }
        if (a.s8) {
          // S in MXFP8 along D: the 32 columns of a scale block are the chunks of 4
          // neighbouring lanes (the exchange runs on every lane; D % 64 == 0 keeps such a group
          // wholly inside or outside the row)
          uint8_t* codes = static_cast<uint8_t*>(a.s8) + size_t(h) * size_t(pk_rows(B)) * D;
          uint8_t* scales = static_cast<uint8_t*>(a.s8_scale) + size_t(h) * size_t(pk_rows(B)) * D / 32;
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            float amax = 0.f;
            if (c < nchunks)
#pragma unroll
              for (int e = 0; e < W; ++e) amax = fmaxf(amax, fabsf(r[i][e]));
            amax = quad_max(amax);
            const uint32_t sb = mx_scale_bits(amax);
            const float inv = mx_inv_scale(sb);
            if (c < nchunks) {
              float v[W];
#pragma unroll
              for (int e = 0; e < W; ++e) v[e] = r[i][e] * inv;
              const int col = c * W;
              *reinterpret_cast<uint2*>(codes + mx_off(b, col, D) + ((col >> 3) & 1) * 8) = e4m3_pack8(v);
              if ((lane & 3) == 0) scales[mx_scale_off(b, col >> 5, D)] = uint8_t(sb);
            }
          }
        }
        continue;
      }
    }
    T* dst = static_cast<T*>(a.S) + (size_t(h) * B + b) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunks) storew<W>(dst + c * W, r[i]);
    }
  }
}

// Standalone Token Mixing: Y[b, h, c] = X[b, t, mix_source(h, c)], W columns per thread.
template <typename T, int W>
__global__ __launch_bounds__(256) void token_mix_kernel(const T* __restrict__ X, T* __restrict__ Y,
                                                        int64_t total, int Tn, int D) {
  const int q = D / Tn;
  const int per_row = D / W;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int c = int(i % per_row) * W;
    const int64_t bh = i / per_row;
    const int h = int(bh % Tn);
    const int64_t b = bh / Tn;
    int t;
    const int sc = mix_source(h, c, q, &t);
    const T* src = X + (b * Tn + t) * D + sc;
    T* dst = Y + bh * D + c;
    if constexpr (W == 8) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      if constexpr (sizeof(T) == 4) reinterpret_cast<uint4*>(dst)[1] = reinterpret_cast<const uint4*>(src)[1];
    } else {
      *dst = *src;
    }
  }
}

template <typename T, int W, int NC>
hipError_t launch_rows_nc(int mode, const RowsArgs& a, hipStream_t stream) {
  const bool moe = a.moe_ye != nullptr;
  if (moe && (sizeof(T) != 2 || mode == ROWS_FIRST)) return hipErrorInvalidValue;
  const int maxw = rows_max_waves(NC, mode, moe);
  int nw = a.T < maxw ? a.T : maxw;
  size_t lds;
  if (mode == ROWS_FINAL) {
    while (nw > 1 && size_t(nw) * a.D * 4 > 64 * 1024) --nw;
    lds = size_t(nw) * a.D * 4;
  } else {
    lds = size_t(a.T) * a.D * sizeof(T);
  }
  dim3 grid(a.B), block(64 * nw);
  if constexpr (sizeof(T) == 2) {
    if (moe) {
      if (mode == ROWS_MID)
        hipLaunchKernelGGL((rows_kernel<T, W, NC, ROWS_MID, true>), grid, block, lds, stream, a);
      else
        hipLaunchKernelGGL((rows_kernel<T, W, NC, ROWS_FINAL, true>), grid, block, lds, stream, a);
      return hipGetLastError();
    }
  }
  switch (mode) {
    case ROWS_FIRST:
      hipLaunchKernelGGL((rows_kernel<T, W, NC, ROWS_FIRST>), grid, block, lds, stream, a);
      break;
    case ROWS_MID:
      hipLaunchKernelGGL((rows_kernel<T, W, NC, ROWS_MID>), grid, block, lds, stream, a);
      break;
    default:
      hipLaunchKernelGGL((rows_kernel<T, W, NC, ROWS_FINAL>), grid, block, lds, stream, a);
      break;
  }
  return hipGetLastError();
}

// chunks per lane: ceil(D / (64 W)); the scalar path (small D) always takes 8
template <typename T, int W>
hipError_t launch_rows_t(int mode, const RowsArgs& a, hipStream_t stream) {
  if constexpr (W == 1) {
    return launch_rows_nc<T, 1, ROWS_MAX_D_SCALAR / 64>(mode, a, stream);
  } else {
    switch ((a.D / W + 63) / 64) {
      case 1: return launch_rows_nc<T, W, 1>(mode, a, stream);
      case 2: return launch_rows_nc<T, W, 2>(mode, a, stream);
      case 3: return launch_rows_nc<T, W, 3>(mode, a, stream);
      case 4: return launch_rows_nc<T, W, 4>(mode, a, stream);
      case 5: return launch_rows_nc<T, W, 5>(mode, a, stream);
      case 6: return launch_rows_nc<T, W, 6>(mode, a, stream);
      case 7: return launch_rows_nc<T, W, 7>(mode, a, stream);
      default: return launch_rows_nc<T, W, 8>(mode, a, stream);
    }
  }
}

template <typename T, int W, int NC>
hipError_t set_rows_lds_limit_nc() {
  const int bytes = int(ROWS_MAX_LDS);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_kernel<T, W, NC, ROWS_FIRST>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_kernel<T, W, NC, ROWS_MID>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if constexpr (sizeof(T) == 2) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_kernel<T, W, NC, ROWS_MID, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_kernel<T, W, NC, ROWS_FINAL, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&rows_kernel<T, W, NC, ROWS_FINAL>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename T>
hipError_t set_rows_lds_limit() {
  hipError_t e;
  if ((e = set_rows_lds_limit_nc<T, 1, ROWS_MAX_D_SCALAR / 64>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 1>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 2>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 3>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 4>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 5>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 6>()) != hipSuccess) return e;
  if ((e = set_rows_lds_limit_nc<T, 8, 7>()) != hipSuccess) return e;
  return set_rows_lds_limit_nc<T, 8, 8>();
}

}  // namespace

bool rows_vectorized(int T, int D) { return D % 8 == 0 && (D / T) % 8 == 0; }

size_t rows_lds_bytes(int dtype, int T, int D) { return size_t(T) * D * dtype_size(dtype); }

hipError_t rows_init() {
  hipError_t e = set_rows_lds_limit<float>();
  if (e != hipSuccess) return e;
  return set_rows_lds_limit<bf16_t>();
}

hipError_t launch_rows(int dtype, int mode, const RowsArgs& a, hipStream_t stream) {
  const bool vec = rows_vectorized(a.T, a.D);
  if (dtype == DT_BF16)
    return vec ? launch_rows_t<bf16_t, 8>(mode, a, stream) : launch_rows_t<bf16_t, 1>(mode, a, stream);
  return vec ? launch_rows_t<float, 8>(mode, a, stream) : launch_rows_t<float, 1>(mode, a, stream);
}

hipError_t launch_token_mix(int dtype, const void* X, void* Y, int64_t B, int T, int D,
                            hipStream_t stream) {
  const bool vec = rows_vectorized(T, D);
  const int W = vec ? 8 : 1;
  const int64_t total = B * T * (D / W);
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 65536 ? want : 65536);
  if (dtype == DT_BF16) {
    if (vec)
      hipLaunchKernelGGL((token_mix_kernel<bf16_t, 8>), dim3(blocks), dim3(256), 0, stream,
                         static_cast<const bf16_t*>(X), static_cast<bf16_t*>(Y), total, T, D);
    else
      hipLaunchKernelGGL((token_mix_kernel<bf16_t, 1>), dim3(blocks), dim3(256), 0, stream,
                         static_cast<const bf16_t*>(X), static_cast<bf16_t*>(Y), total, T, D);
  } else {
    if (vec)
      hipLaunchKernelGGL((token_mix_kernel<float, 8>), dim3(blocks), dim3(256), 0, stream,
                         static_cast<const float*>(X), static_cast<float*>(Y), total, T, D);
    else
      hipLaunchKernelGGL((token_mix_kernel<float, 1>), dim3(blocks), dim3(256), 0, stream,
                         static_cast<const float*>(X), static_cast<float*>(Y), total, T, D);
  }
  return hipGetLastError();
}

}  // namespace rmx
