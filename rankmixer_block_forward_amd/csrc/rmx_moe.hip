// Sparse-MoE per-token FFN: ReLU router and token -> expert row lists.
// RankMixer paper translation, section 3.4 eq (10): for token t with its own E experts,
// G = ReLU(h(s_t)) and v_t = sum_e G_e * expert_e(s_t); an expert whose gate is zero is
// not evaluated.  The expert FFNs themselves run as grouped GEMMs (rmx_gemm.hip) over the
// compacted row lists built here, one group per (token, expert).
//
// Group gi = t * E + e.  All lists are deterministic: rows of a group appear in ascending
// sample order.  The combine (S plus the gate-scaled expert rows, in expert order) runs in
// the next row pass (rmx_rows.hip).
#include "rmx_device.h"
#include "rmx_internal.h"

namespace rmx {

namespace {

// Gate: g[t][e][b] = max(0, S[t][b] . Wg[t][:, e]) in fp32; counts of active rows per
// (t, e, 64-row chunk).  Grid (ceil(B / 256), T), 256 threads: lane l of wave w owns sample
// row b = 256 blockIdx.x + 64 w + l, which it streams in 16-byte pieces, so a wave covers
// exactly one 64-row chunk and its counts are one ballot per expert.  Wg[t] is staged in
// LDS as fp32, element (d, e) at d * EP + e (EP = E rounded up to 4, zero padded); every
// lane of a wave reads the same weights at the same time (LDS broadcast).  The dot product
// runs over d in order.  D % 32 == 0 (the expert products' K step).
__host__ __device__ constexpr int gate_ep(int E) { return (E + 3) & ~3; }

template <int EP>
__global__ __launch_bounds__(256) void moe_gate_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float wg[];
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D, E = a.E, B = a.B, T = a.T;
  // Wg[t] ([D][E] bf16, contiguous, D * E % 8 == 0): 16-byte loads, fp32 into LDS
  const bf16_t* Wg = static_cast<const bf16_t*>(a.Wg) + size_t(t) * D * E;
  for (int i = threadIdx.x; i < D * E / 8; i += blockDim.x) {
    float v[8];
    load8(Wg + 8 * i, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = 8 * i + u, d = idx / E, e = idx - d * E;
      wg[d * EP + e] = v[u];
    }
  }
  if (E < EP)
    for (int i = threadIdx.x; i < D * (EP - E); i += blockDim.x) {
      const int d = i / (EP - E), e = E + (i - d * (EP - E));
      wg[d * EP + e] = 0.f;
    }
  __syncthreads();
  const int chunk = blockIdx.x * 4 + wave;
  if (chunk >= a.nchunk) return;  // no barrier follows
  const int b = chunk * 64 + lane;
  const bool in = b < B;
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.f;
  if (in) {
    const bf16_t* srow = static_cast<const bf16_t*>(a.S) + (size_t(t) * B + b) * D;
    // four 16-byte pieces in flight per step (D % 32 == 0 on this path)
    for (int c0 = 0; c0 < D / 8; c0 += 4) {
      float v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) load8(srow + (c0 + j) * 8, v[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* wb = wg + (c0 + j) * 8 * EP;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e4 = 0; e4 < EP; e4 += 4) {
            const float4 w = *reinterpret_cast<const float4*>(wb + u * EP + e4);
            acc[e4 + 0] = fmaf(v[j][u], w.x, acc[e4 + 0]);
            acc[e4 + 1] = fmaf(v[j][u], w.y, acc[e4 + 1]);
            acc[e4 + 2] = fmaf(v[j][u], w.z, acc[e4 + 2]);
            acc[e4 + 3] = fmaf(v[j][u], w.w, acc[e4 + 3]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    if (e >= E) break;
    const float gv = acc[e] > 0.f ? acc[e] : 0.f;
    if (in) {
      a.g[(size_t(t) * E + e) * B + b] = gv;
      if (a.gate_out) a.gate_out[(size_t(b) * T + t) * E + e] = gv;
    }
    const uint64_t m = __ballot(in && gv > 0.f);
    if (lane == 0) a.cnt[(size_t(t) * E + e) * a.nchunk + chunk] = __popcll(m);
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

}  // namespace

size_t moe_gate_lds_bytes(int D, int E) { return size_t(D) * gate_ep(E) * sizeof(float); }

hipError_t moe_init() {
  const int bytes = int(MOE_MAX_GATE_LDS);
  hipError_t e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_gate_kernel<4>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_gate_kernel<8>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_gate_kernel<12>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess)
    return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_gate_kernel<16>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_moe_route(const MoeArgs& a, hipStream_t stream) {
  const size_t lds = moe_gate_lds_bytes(a.D, a.E);
  const dim3 grid((a.nchunk + 3) / 4, a.T);
  switch (gate_ep(a.E)) {
    case 4: hipLaunchKernelGGL((moe_gate_kernel<4>), grid, dim3(256), lds, stream, a); break;
    case 8: hipLaunchKernelGGL((moe_gate_kernel<8>), grid, dim3(256), lds, stream, a); break;
    case 12: hipLaunchKernelGGL((moe_gate_kernel<12>), grid, dim3(256), lds, stream, a); break;
    default: hipLaunchKernelGGL((moe_gate_kernel<16>), grid, dim3(256), lds, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(a.nchunk, a.T), dim3(64), 0, stream, a);
  return hipGetLastError();
}


}  // namespace rmx
