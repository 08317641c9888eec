// Sparse-MoE per-token FFN: ReLU router, token -> expert row lists, combine.
// RankMixer paper translation, section 3.4 eq (10): for token t with its own E experts,
// G = ReLU(h(s_t)) and v_t = sum_e G_e * expert_e(s_t); an expert whose gate is zero is
// not evaluated.  The expert FFNs themselves run as grouped GEMMs (rmx_gemm.hip) over the
// compacted row lists built here, one group per (token, expert).
//
// Group gi = t * E + e.  All lists are deterministic: rows of a group appear in ascending
// sample order, and the combine sums the experts of a row in expert order.
#include "rmx_device.h"
#include "rmx_internal.h"

namespace rmx {

namespace {

// Gate: g[t][e][b] = max(0, S[t][b] . Wg[t][:, e]) in fp32; counts of active rows per
// (t, e, 64-row chunk).  Grid (chunks, T), 256 threads: wave w handles rows 16 w .. 16 w + 15
// of the chunk, one row at a time, each lane taking 8-element pieces of the row.  Wg[t] is
// staged in LDS transposed to [E][D] so that each lane reads 32 contiguous bytes per expert.
__global__ __launch_bounds__(256) void moe_gate_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) float wg[MOE_MAX_GATE_WEIGHTS];
  __shared__ int wave_cnt[4][MOE_MAX_E];
  const int t = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D, E = a.E, B = a.B, T = a.T;
  const bf16_t* Wg = static_cast<const bf16_t*>(a.Wg) + size_t(t) * D * E;
  for (int i = threadIdx.x; i < D * E; i += blockDim.x) {
    const int d = i / E, e = i - d * E;
    wg[e * D + d] = load1(Wg + i);
  }
  __syncthreads();
  int my_cnt = 0;  // lane e (< E) counts the active rows of expert e in this wave
  for (int rr = 0; rr < 16; ++rr) {
    const int b = chunk * 64 + wave * 16 + rr;
    if (b >= B) break;  // uniform within the wave
    const bf16_t* s = static_cast<const bf16_t*>(a.S) + (size_t(t) * B + b) * D;
    float acc[MOE_MAX_E];
#pragma unroll
    for (int e = 0; e < MOE_MAX_E; ++e) acc[e] = 0.f;
    for (int c = lane; c < D / 8; c += 64) {
      float v[8];
      load8(s + c * 8, v);
#pragma unroll
      for (int e = 0; e < MOE_MAX_E; ++e) {
        if (e < E) {
          const float4 w0 = *reinterpret_cast<const float4*>(wg + e * D + c * 8);
          const float4 w1 = *reinterpret_cast<const float4*>(wg + e * D + c * 8 + 4);
          float r = acc[e];
          r = fmaf(v[0], w0.x, r); r = fmaf(v[1], w0.y, r); r = fmaf(v[2], w0.z, r); r = fmaf(v[3], w0.w, r);
          r = fmaf(v[4], w1.x, r); r = fmaf(v[5], w1.y, r); r = fmaf(v[6], w1.z, r); r = fmaf(v[7], w1.w, r);
          acc[e] = r;
        }
      }
    }
    float mine = 0.f;
#pragma unroll
    for (int e = 0; e < MOE_MAX_E; ++e) {
      if (e < E) {
        const float tot = wave_sum(acc[e]);
        if (lane == e) mine = tot;
      }
    }
    if (lane < E) {
      const float gv = mine > 0.f ? mine : 0.f;
      a.g[(size_t(t) * E + lane) * B + b] = gv;
      if (a.gate_out) a.gate_out[(size_t(b) * T + t) * E + lane] = gv;
      my_cnt += gv > 0.f ? 1 : 0;
    }
  }
  if (lane < E) wave_cnt[wave][lane] = my_cnt;
  __syncthreads();
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    a.cnt[(size_t(t) * E + e) * a.nchunk + chunk] =
        wave_cnt[0][e] + wave_cnt[1][e] + wave_cnt[2][e] + wave_cnt[3][e];
  }
}

// Scan (one workgroup): chunk offsets within each group, group row offsets, and the
// cumulative count of 256-row tiles per group.  Thread gi owns group gi.
__global__ __launch_bounds__(1024) void moe_scan_kernel(MoeArgs a) {
  __shared__ int part[1024];
  const int G = a.T * a.E;
  int total = 0, tiles = 0;
  for (int gi = threadIdx.x; gi < G; gi += blockDim.x) {
    // each thread owns at most one group (G <= 1024, checked on the host)
    int run = 0;
    int* c = a.cnt + size_t(gi) * a.nchunk;
    int* off = a.chunk_off + size_t(gi) * a.nchunk;
    for (int k = 0; k < a.nchunk; ++k) {
      off[k] = run;
      run += c[k];
    }
    a.group_rows[gi] = run;
    total = run;
    tiles = (run + MOE_TILE_M - 1) / MOE_TILE_M;
  }
  // exclusive scan over groups of (rows, tiles), in group order
  part[threadIdx.x] = total;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  if (threadIdx.x < G) a.group_start[threadIdx.x] = part[threadIdx.x] - total;
  if (threadIdx.x == G - 1) a.group_start[G] = part[threadIdx.x];
  __syncthreads();
  part[threadIdx.x] = threadIdx.x < G ? tiles : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  if (threadIdx.x < G) a.tile_start[threadIdx.x] = part[threadIdx.x] - tiles;
  if (threadIdx.x == G - 1) a.tile_start[G] = part[threadIdx.x];
}

// Scatter (one wave per 64-row chunk of token t): the compacted position of every active
// (t, e, b), its source row in S, its gate value, and the inverse map pos[t][e][b].
__global__ __launch_bounds__(64) void moe_scatter_kernel(MoeArgs a) {
  const int t = blockIdx.y, chunk = blockIdx.x, lane = threadIdx.x;
  const int b = chunk * 64 + lane;
  const bool in = b < a.B;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < a.E; ++e) {
    const int gi = t * a.E + e;
    const float gv = in ? a.g[size_t(gi) * a.B + b] : 0.f;
    const bool act = gv > 0.f;
    const uint64_t mask = __ballot(act);
    if (in) {
      int pos = -1;
      if (act) {
        pos = a.group_start[gi] + a.chunk_off[size_t(gi) * a.nchunk + chunk] + __popcll(mask & below);
        a.src_row[pos] = t * a.B + b;
        a.row_gate[pos] = gv;
      }
      a.pos[size_t(gi) * a.B + b] = pos;
    }
  }
}

// Combine: Y[t][b] = S[t][b] + sum_e (active ? Ye[pos[t][e][b]] : 0), experts in order.
// Ye rows already carry their gate factor.  One 64-lane wave per (t, b) row.
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;  // row = t * B + b
  if (row >= int64_t(a.T) * a.B) return;
  const int t = int(row / a.B), b = int(row % a.B);
  const int D = a.D;
  const bf16_t* s = static_cast<const bf16_t*>(a.S) + size_t(row) * D;
  float* y = a.Y + size_t(row) * D;
  for (int c = lane; c < D / 8; c += 64) {
    float acc[8];
    load8(s + c * 8, acc);
    for (int e = 0; e < a.E; ++e) {
      const int pos = a.pos[size_t(t * a.E + e) * a.B + b];
      if (pos >= 0) {
        float v[8];
        load8(a.Ye + size_t(pos) * D + c * 8, v);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += v[u];
      }
    }
    store8(y + c * 8, acc);
  }
}

}  // namespace

hipError_t launch_moe_route(const MoeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(moe_gate_kernel, dim3(a.nchunk, a.T), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(a.nchunk, a.T), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const MoeArgs& a, hipStream_t stream) {
  const int64_t rows = int64_t(a.T) * a.B;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rmx
