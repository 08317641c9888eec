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
// (t, e, 64-row chunk).  Grid (chunks, T), 256 threads: wave w handles rows 16 w .. 16 w + 15
// of the chunk, 8 rows at a time, each row split over 8 lanes (lane = 8 r + s takes the
// 8-element pieces s, s + 8, ... of row r: the 8 lanes of a row read 128 contiguous bytes).
// Wg[t] is staged in LDS as fp32, element (d, e) at (d / 8) * GATE_BLK + (d % 8) * EP + e with
// EP = E rounded up to 4 (zero padded) and GATE_BLK = 8 EP + 4, so that the 8 pieces read
// in one step fall in distinct banks.  Partial sums meet over the 8 lanes of a row by
// butterfly exchange, in a fixed order.
__host__ __device__ constexpr int gate_ep(int E) { return (E + 3) & ~3; }
__host__ __device__ constexpr int gate_blk(int E) { return 8 * gate_ep(E) + 4; }

template <int EP>
__global__ __launch_bounds__(256) void moe_gate_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float wg[];
  __shared__ int wave_cnt[4][MOE_MAX_E];
  const int t = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D, E = a.E, B = a.B, T = a.T;
  constexpr int BLK = 8 * EP + 4;
  const bf16_t* Wg = static_cast<const bf16_t*>(a.Wg) + size_t(t) * D * E;
  for (int i = threadIdx.x; i < D * EP; i += blockDim.x) {
    const int d = i / EP, e = i - d * EP;
    wg[(d >> 3) * BLK + (d & 7) * EP + e] = e < E ? load1(Wg + d * E + e) : 0.f;
  }
  __syncthreads();
  const int r = lane >> 3, sl = lane & 7;
  const int nch = D / 8;
  int my_cnt[MOE_MAX_E];  // active rows of expert e in this wave (uniform)
#pragma unroll
  for (int e = 0; e < MOE_MAX_E; ++e) my_cnt[e] = 0;
  for (int grp = 0; grp < 2; ++grp) {
    const int b = chunk * 64 + wave * 16 + grp * 8 + r;
    const bool in = b < B;
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    if (in) {
      const bf16_t* srow = static_cast<const bf16_t*>(a.S) + (size_t(t) * B + b) * D;
      for (int c = sl; c < nch; c += 8) {
        float v[8];
        load8(srow + c * 8, v);
        const float* wb = wg + c * BLK;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e4 = 0; e4 < EP; e4 += 4) {
            const float4 w = *reinterpret_cast<const float4*>(wb + u * EP + e4);
            acc[e4 + 0] = fmaf(v[u], w.x, acc[e4 + 0]);
            acc[e4 + 1] = fmaf(v[u], w.y, acc[e4 + 1]);
            acc[e4 + 2] = fmaf(v[u], w.z, acc[e4 + 2]);
            acc[e4 + 3] = fmaf(v[u], w.w, acc[e4 + 3]);
          }
        }
      }
    }
    // sum over the 8 lanes of the row (every lane ends with all totals)
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float x = acc[e];
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      acc[e] = x;
    }
    // lane s of the row writes experts s and s + 8
#pragma unroll
    for (int h = 0; h < (EP + 7) / 8; ++h) {
      const int e = sl + 8 * h;
      float tot = 0.f;
#pragma unroll
      for (int k = 0; k < EP; ++k)
        if (k == e) tot = acc[k];
      const float gv = tot > 0.f ? tot : 0.f;
      const bool act = in && e < E && gv > 0.f;
      if (in && e < E) {
        a.g[(size_t(t) * E + e) * B + b] = gv;
        if (a.gate_out) a.gate_out[(size_t(b) * T + t) * E + e] = gv;
      }
      const uint64_t m = __ballot(act);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (8 * h + k < MOE_MAX_E) my_cnt[8 * h + k] += __popcll(m & (0x0101010101010101ull << k));
    }
  }
  if (lane == 0)
#pragma unroll
    for (int e = 0; e < MOE_MAX_E; ++e)
      if (e < E) wave_cnt[wave][e] = my_cnt[e];
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

}  // namespace

size_t moe_gate_lds_bytes(int D, int E) { return size_t(D / 8) * gate_blk(E) * sizeof(float); }

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
  const dim3 grid(a.nchunk, a.T);
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
