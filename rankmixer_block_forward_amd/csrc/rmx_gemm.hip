// Grouped GEMMs of the per-token FFN: token t multiplies its rows S[t] (or the hidden
// activations) by its own weights, all T products in one launch.
// RankMixer paper translation, section 3.3.2 eq (6)-(9) (per-token FFN) and section
// 4.6 (the parallel per-token FFNs fused into one operator); "RankMixer 详解（1）",
// section 4.3 (the batch rows share each token's weights).
//
// Two kernels:
//   gemm_bf16_mfma  bf16 inputs, fp32 accumulation on the CDNA4 matrix cores
//                   (v_mfma_f32_32x32x16_bf16).  Needs K % 64 == 0 and N % 8 == 0;
//                   any M (rows past M are zero-filled and never stored).
//   gemm_generic    any shape, fp32 or bf16 inputs, fp32 FMA on the vector ALUs
//                   (the fp32 path and shapes the MFMA kernel does not take).
// Epilogues: EPI_GELU writes GELU(acc + bias) in the input dtype (the hidden
// activations); EPI_RESID writes acc + bias + R in fp32 (the pre-LN2 rows).
#include "rmx_device.h"
#include "rmx_internal.h"

namespace rmx {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ MFMA kernel
// Workgroup tile 256 x 256, K step 64, 4 waves in a 2 x 2 grid, each wave 128 x 128 as
// 4 x 4 blocks of 32 x 32 MFMA accumulators (256 fp32 accumulator registers per lane).
// Both operands are staged through LDS with the reduction index K contiguous: A rows as
// they are in memory, W (stored K x N, N contiguous) transposed 8 x 8 in registers on
// the way in.  LDS rows are padded to 72 elements (144 B) so that the 16-byte fragment
// reads of 8 or 16 consecutive rows fall in distinct banks.  Two LDS stages: the global
// loads of step i+1 are in flight while step i runs on the matrix cores.
constexpr int BM = 256, BN = 256, BK = 64, LDK = 72;
constexpr int A_STAGE = BM * LDK;  // elements
constexpr int B_STAGE = BN * LDK;
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int MFMA_THREADS = 256;
constexpr int EPI_LD = 132;        // fp32 row stride of the epilogue staging tile
constexpr int NUM_XCD = 8;         // MI355X: 8 accelerator complex dies, each with its own L2

// Workgroups are dealt to the XCDs round-robin.  Remap so that each XCD receives a
// contiguous range of tile indices, and order tiles M-fastest within a token so that the
// tiles resident on one XCD at a time share their weight panels and A rows in its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % NUM_XCD, pos = bid / NUM_XCD;
  const int base = nblocks / NUM_XCD, extra = nblocks % NUM_XCD;
  return xcd * base + (xcd < extra ? xcd : extra) + pos;
}

template <int EPI>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_mfma(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = (N + BN - 1) / BN;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  const int nt = rem / nMt, mt = rem - nt * nMt;
  const int m0 = mt * BM, n0 = nt * BN;

  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(p.A) + size_t(g) * M * K;
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(p.W) + size_t(g) * K * N;

  // Global -> register mapping.  A: 16 B chunk ac (8 consecutive k) of rows ar + 32 i.
  // W: rows wk0 .. wk0+7 (k) of the 8 columns starting at wn0 (n).
  const int ac = tid & 7, ar = tid >> 3;
  const int wkg = tid & 7, wnc = tid >> 3;
  const int wn0 = n0 + wnc * 8;
  const bool wcol_ok = wn0 < N;
  uint4 ra[8];
  uint32_t rb[8][4];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = m0 + ar + 32 * i;
      if (row < M)
        ra[i] = *reinterpret_cast<const uint4*>(A + size_t(row) * K + k0 + ac * 8);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (wcol_ok) v = *reinterpret_cast<const uint4*>(W + size_t(k0 + wkg * 8 + i) * N + wn0);
      rb[i][0] = v.x; rb[i][1] = v.y; rb[i][2] = v.z; rb[i][3] = v.w;
    }
  };

  auto lstore = [&](int stage) {
    uint16_t* As = smem + stage * STAGE;
    uint16_t* Bs = As + A_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(As + (ar + 32 * i) * LDK + ac * 8) = ra[i];
    // 8 x 8 transpose: rb[i] holds W[k = i][n = 0..7] as 4 words of 2 bf16; column n of
    // the result holds k = 0..7, word u = (k = 2u) | (k = 2u + 1) << 16.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint4 lo, hi;  // columns n = 2w (low halves) and n = 2w + 1 (high halves)
      lo.x = __builtin_amdgcn_perm(rb[1][w], rb[0][w], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(rb[3][w], rb[2][w], 0x05040100u);
      lo.z = __builtin_amdgcn_perm(rb[5][w], rb[4][w], 0x05040100u);
      lo.w = __builtin_amdgcn_perm(rb[7][w], rb[6][w], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(rb[1][w], rb[0][w], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(rb[3][w], rb[2][w], 0x07060302u);
      hi.z = __builtin_amdgcn_perm(rb[5][w], rb[4][w], 0x07060302u);
      hi.w = __builtin_amdgcn_perm(rb[7][w], rb[6][w], 0x07060302u);
      *reinterpret_cast<uint4*>(Bs + (wnc * 8 + 2 * w) * LDK + wkg * 8) = lo;
      *reinterpret_cast<uint4*>(Bs + (wnc * 8 + 2 * w + 1) * LDK + wkg * 8) = hi;
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) gload((it + 1) * BK);
    const uint16_t* As = smem + cur * STAGE;
    const uint16_t* Bs = As + A_STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // MFMA 32x32x16 operand layout: lane l supplies row (l % 32) of A and column
      // (l % 32) of B, each with the 8 consecutive k at 8 * (l / 32) of this 16-k step.
      const int kc = kk * 16 + (lane >> 5) * 8;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 128 + i * 32 + (lane & 31)) * LDK + kc);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 128 + j * 32 + (lane & 31)) * LDK + kc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator layout of a 32 x 32 block: lane l, register r holds
  // row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  Each wave stages 32 rows x 128
  // columns at a time through LDS so that every lane then owns 8 consecutive columns of
  // one row: 16-byte global stores, and coalesced bias / residual loads.
  float* st = reinterpret_cast<float*>(smem) + wave * 32 * EPI_LD;
  const int col8 = (lane & 15) * 8;
  const int rsub = lane >> 4;
  const int n = n0 + wn * 128 + col8;
  const bool n_ok = n < N;
  float bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bias[e] = 0.f;
  if (p.bias && n_ok) load8(static_cast<const bf16_t*>(p.bias) + size_t(g) * N + n, bias);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        st[row * EPI_LD + j * 32 + (lane & 31)] = acc[i][j][r];
      }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int row = pass * 4 + rsub;
      const int m = m0 + wm * 128 + i * 32 + row;
      float v[8];
      const float4 x0 = *reinterpret_cast<const float4*>(st + row * EPI_LD + col8);
      const float4 x1 = *reinterpret_cast<const float4*>(st + row * EPI_LD + col8 + 4);
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
      v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      if (m < M && n_ok) {
        const size_t off = (size_t(g) * M + m) * N + n;
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_exact(v[e] + bias[e]);
          store8(static_cast<bf16_t*>(p.C) + off, v);
        } else {
          float rr[8];
          load8(static_cast<const bf16_t*>(p.R) + off, rr);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] + bias[e] + rr[e];
          store8(static_cast<float*>(p.C) + off, v);
        }
      }
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- generic kernel
// 64 x 64 tile, K step 16, 256 threads each computing 4 x 4 outputs in fp32.
constexpr int GT = 64, GK = 16;

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_generic(GemmArgs p) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int M = p.M, N = p.N, K = p.K;
  const int g = blockIdx.z;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const T* A = static_cast<const T*>(p.A) + size_t(g) * M * K;
  const T* W = static_cast<const T*>(p.W) + size_t(g) * K * N;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += GK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;  // 0..1023
      const int am = e / GK, ak = e % GK;
      const int row = m0 + am, kk = k0 + ak;
      As[ak][am] = (row < M && kk < K) ? load1(A + size_t(row) * K + kk) : 0.f;
      const int bk = e / GT, bn = e % GT;
      const int kr = k0 + bk, col = n0 + bn;
      Bs[bk][bn] = (kr < K && col < N) ? load1(W + size_t(kr) * N + col) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float bias = p.bias ? load1(static_cast<const T*>(p.bias) + size_t(g) * N + n) : 0.f;
      const size_t off = (size_t(g) * M + m) * N + n;
      if constexpr (EPI == EPI_GELU) {
        store1(static_cast<T*>(p.C) + off, gelu_exact(acc[i][j] + bias));
      } else {
        static_cast<float*>(p.C)[off] = acc[i][j] + bias + load1(static_cast<const T*>(p.R) + off);
      }
    }
  }
}

}  // namespace

bool gemm_uses_mfma(int dtype, int N, int K) { return dtype == DT_BF16 && K % BK == 0 && N % 8 == 0; }

hipError_t gemm_init() { return hipSuccess; }

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t stream) {
  if (a.G == 0 || a.M == 0 || a.N == 0) return hipSuccess;
  if (gemm_uses_mfma(dtype, a.N, a.K)) {
    const int tiles = a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_GELU>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_RESID>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid((a.N + GT - 1) / GT, (a.M + GT - 1) / GT, a.G);
  if (dtype == DT_BF16) {
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_generic<bf16_t, EPI_GELU>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_generic<bf16_t, EPI_RESID>), grid, dim3(256), 0, stream, a);
  } else {
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_generic<float, EPI_GELU>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_generic<float, EPI_RESID>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rmx
