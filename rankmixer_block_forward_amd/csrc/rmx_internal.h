// Host-side interface between the C ABI layer (rmx_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmx_layout.h"

namespace rmx {

enum Dtype { DT_FP32 = 0, DT_BF16 = 1 };

inline int dtype_size(int dt) { return dt == DT_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- row kernel
// One workgroup per sample.  Modes:
//   ROWS_FIRST  in = X0 [B, T, D] (dtype): S = LN1(mix(X0) + X0)
//   ROWS_MID    in = Y  [T, B, D] (fp32, pre-LN2 rows of the previous block):
//               X = LN2(Y); S = LN1(mix(X) + X)
//   ROWS_FINAL  in = Y: X_L = LN2(Y); pool[b] = mean_t X_L[b, t]; xl (optional) = X_L
// S is written token-major [T, B, D] (dtype), the layout the grouped GEMMs read.
enum RowsMode { ROWS_FIRST = 0, ROWS_MID = 1, ROWS_FINAL = 2 };


struct RowsArgs {
  const void* in;
  const void* ln2_g;
  const void* ln2_b;
  const void* ln1_g;
  const void* ln1_b;
  void* S;
  float* pool;
  void* xl;
  int B, T, D;
  float eps;
  int s_packed;  // S in the packed operand layout, token t at S + t * pk_rows(B) * D
  // With s_packed: also S in MXFP8 (token t's codes at s8 + t * pk_rows(B) * D bytes, its
  // scales at s8_scale + t * pk_rows(B) * D / 32 bytes), nullable
  void* s8;
  void* s8_scale;
  // ROWS_MID / ROWS_FINAL after a Sparse-MoE block (moe_ye non-null): the pre-LN2 rows are
  // formed on the fly, Y[t, b] = S[t, b] + sum over e in order of Ye[pos[t][e][b]] (fp32,
  // experts with pos < 0 skipped), with in = that block's S [T, B, D] (bf16), moe_ye its
  // gate-scaled expert rows [rows, D] (bf16) and moe_pos [T * E][B].
  const void* moe_ye;
  const int* moe_pos;
  int moe_E;
};

// Largest D the row kernel's per-lane registers hold.
constexpr int ROWS_MAX_D = 4096;
constexpr int ROWS_MAX_D_SCALAR = 512;
// On-chip bytes one sample needs in the row kernel (ROWS_FIRST / ROWS_MID).
size_t rows_lds_bytes(int dtype, int T, int D);
constexpr size_t ROWS_MAX_LDS = 96 * 1024;
bool rows_vectorized(int T, int D);

// Once per process and device, before the first launch (raises the LDS limit).
hipError_t rows_init();
hipError_t launch_rows(int dtype, int mode, const RowsArgs& a, hipStream_t stream);
hipError_t launch_token_mix(int dtype, const void* X, void* Y, int64_t B, int T, int D,
                            hipStream_t stream);

// ---------------------------------------------------------------- backward row kernel
// One workgroup per sample ("RankMixer 详解（1）", section 5.2).  Modes:
//   BWD_TOP     gY = LN2_backward(g_out / T) of the last block (Y = its pre-LN2 rows)
//   BWD_MID     X = LN2(Y) of block n - 1 recomputed in LDS; gR = LN1_backward(gS) of block
//               n; gX = gR + P^T gR; gY = LN2_backward(gX) of block n - 1
//   BWD_BOTTOM  X = X0; gR = LN1_backward(gS) of block 1; dX = gR + P^T gR
enum RowsBwdMode { BWD_TOP = 0, BWD_MID = 1, BWD_BOTTOM = 2 };

struct RowsBwdArgs {
  const void* X0;      // BOTTOM: [B, T, D] (dtype), the stack input
  const float* Y;      // TOP, MID: [T, B, D] pre-LN2 rows (of block L, of block n - 1)
  const void* ln2_g;   // TOP, MID: LN2 gamma / beta of that block [D] (dtype)
  const void* ln2_b;
  const void* ln1_g;   // MID, BOTTOM: LN1 gamma of block n [D] (dtype)
  const float* gS;     // MID, BOTTOM: [T, B, D] gradient of block n's S (residual included)
  float* gR;           // MID, BOTTOM: [B, T, D] scratch
  const float* g_out;  // TOP: [B, D] gradient of the pooled output
  float* gY32;         // TOP, MID: [T, B, D] gradient of the pre-LN2 rows (fp32)
  void* gY;            // TOP, MID: the same in dtype (a GEMM operand)
  float* dX;           // BOTTOM: [B, T, D]
  float* part_ln1;     // MID, BOTTOM: [2][B][D] per-sample gamma / beta gradients of LN1
  float* part_ln2;     // TOP, MID: [2][B][D] per-sample gamma / beta gradients of LN2
  int B, T, D;
  float eps;
};

constexpr int ROWS_BWD_MAX_D = 2048;        // vectorized path (D % 8 == 0, (D / T) % 8 == 0)
constexpr int ROWS_BWD_MAX_D_SCALAR = 512;  // scalar path
constexpr size_t ROWS_BWD_MAX_LDS = 128 * 1024;
size_t rows_bwd_lds_bytes(int dtype, int T, int D);
bool rows_bwd_supported(int dtype, int T, int D);
// Once per process and device (raises the kernel's LDS limit).
hipError_t rows_bwd_init();
hipError_t launch_rows_bwd(int dtype, int mode, const RowsBwdArgs& a, hipStream_t stream);

// out[g, n] = sum over r < R of in[g, r, n] (in: dtype, [G, R, N] contiguous; out fp32),
// in a fixed order.  scratch: colsum_scratch_floats(G, R, N) floats.
constexpr int COLSUM_ROWS = 256;
constexpr int COLSUM_MAX_SPLIT = 64;
inline size_t colsum_scratch_floats(int64_t G, int64_t R, int64_t N) {
  int64_t rs = (R + COLSUM_ROWS - 1) / COLSUM_ROWS;
  if (rs > COLSUM_MAX_SPLIT) rs = COLSUM_MAX_SPLIT;
  return size_t(rs > 1 ? rs : 0) * size_t(G) * size_t(N);
}
hipError_t launch_colsum(int dtype, const void* in, float* out, float* scratch, int G, int R, int N,
                         hipStream_t stream);

// ---------------------------------------------------------------- self-attention routing
// The routing comparator: S = LN1(softmax(Q K^T / sqrt(D)) V + X) per sample, one
// workgroup per sample.  Q, K, V, X [B, T, D] (dtype, sample-major); S [T, B, D] (dtype).
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* X;
  const void* ln1_g;
  const void* ln1_b;
  void* S;
  int B, T, D;
  float eps;
};
constexpr int ATTN_MAX_T = 64;     // one key per lane in the softmax
constexpr int ATTN_MAX_D = 2048;   // vectorized path (D % 8 == 0, (D / T) % 8 == 0)
bool attn_supported(int dtype, int T, int D);
hipError_t launch_attn_rows(int dtype, const AttnArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- Sparse-MoE routing
// Group gi = t * E + e.  Rows of a group are listed in ascending sample order.
constexpr int MOE_MAX_E = 16;
constexpr int MOE_MAX_GROUPS = 1024;          // T * E
constexpr int MOE_MAX_GATE_WEIGHTS = 16384;   // D * E (router of one token in LDS)
constexpr size_t MOE_MAX_GATE_LDS = 128 * 1024;  // router LDS (D * E weights, padded)
constexpr int MOE_TILE_M = 256;               // rows per grouped-GEMM tile

struct MoeArgs {
  const void* S;      // [T, B, D] bf16, the LN1 output of this block
  const void* Wg;     // [T, D, E] bf16, router weights of this block
  float* g;           // [T, E, B] gate values
  float* gate_out;    // [B, T, E] of this block, nullable
  int* cnt;           // [T * E, nchunk] active rows per 64-row chunk
  int* chunk_off;     // [T * E, nchunk] exclusive prefix of cnt within a group
  int* group_rows;    // [T * E]
  int* group_start;   // [T * E + 1] first compacted row of each group
  int* tile_start;    // [T * E + 1] cumulative MOE_TILE_M-row tiles
  int* src_row;       // [T * E * B] compacted row -> S row (t * B + b)
  float* row_gate;    // [T * E * B] compacted row -> gate value
  int* pos;           // [T, E, B] -> compacted row, or -1 if the expert is inactive
  int B, T, D, E, nchunk;
};

// Once per process and device (raises the router kernel's LDS limit).
hipError_t moe_init();
// LDS bytes of the router kernel for D columns and E experts.
size_t moe_gate_lds_bytes(int D, int E);
hipError_t launch_moe_route(const MoeArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- grouped GEMM
// G independent products C_g = A_g W_g (+ epilogue), g = 0..G-1 (one per token):
//   A [G, M, K] (dtype)   W [G, K, N] (dtype)   bias [G, N] (dtype, nullable)
//   EPI_GELU:  C [G, M, N] (dtype) = GELU(A W + bias)
//   EPI_RESID: C [G, M, N] (fp32)  = A W + bias + R,  R [G, M, N] (dtype)
//   Sparse-MoE (grouped, variable rows per group, persistent tile loop):
//   EPI_MOE1:  C [rows, N] (bf16) = GELU(A[src_row] W_g + bias_g), A = S [T * B, K]
//   EPI_MOE2:  C [rows, N] (fp32) = row_gate * (A W_g + bias_g),   A = C of EPI_MOE1
//   group g owns compacted rows group_start[g] .. group_start[g + 1] - 1.
//   EPI_BIAS:  C [G, M, N] (dtype) = A W + bias
//   Backward products (no bias):
//   EPI_GELU_BWD: C [G, M, N] (dtype) = (A W) * R,  R [G, M, N] (dtype, GELU' at the
//                 pre-activations, same layout as C)
//   EPI_RESID32:  C [G, M, N] (fp32)  = A W + R,  R [G, M, N] (fp32)
//   EPI_STORE32:  C [G, M, N] (fp32)  = A W
//   With colsum set (matrix-core kernels only), EPI_GELU_BWD also writes the column sums of
//   its fp32 output and EPI_RESID32 those of R, over the 128 rows of each wave:
//   colsum [G, colsum_rows(M), N] fp32, row 2 * (row tile) + (row half of the tile).
//   Training forward:
//   EPI_GELU_SAVE: EPI_GELU that also stores GELU'(A W + bias) in U
//                  ([G, M, N], dtype, C's layout; row-major operands only)
//   MXFP8 products (launch_gemm_mx; A, W and their scales in the MXFP8 layout):
//   EPI_GELU_MX: C = GELU(A W + bias) quantized to MXFP8 along N: codes in C, scales in
//                C_scale ([G][pk_rows(M) x N], the A operand of the second product)
//   EPI_RESID as above (R in the packed bf16 layout).
enum Epilogue {
  EPI_GELU = 0, EPI_RESID = 1, EPI_MOE1 = 2, EPI_MOE2 = 3, EPI_BIAS = 4,
  EPI_GELU_BWD = 5, EPI_RESID32 = 6, EPI_STORE32 = 7, EPI_GELU_SAVE = 8, EPI_GELU_MX = 9
};

constexpr int GEMM_PACKED_W = 2;  // GemmArgs::packed: prepared W^T, row-major A

struct GemmArgs {
  const void* A;
  const void* W;
  const void* bias;
  const void* R;
  void* C;
  int G, M, N, K;
  const int* group_start;
  const int* tile_start;
  const int* src_row;
  const float* row_gate;
  int a_rows;  // EPI_MOE1: rows of A (T * B)
  // Dense kernels only (0 = contiguous): elements between rows of A, between rows of C
  // (and R), between groups of A, between groups of C (and R).
  int64_t lda, ldc, sa, sc;
  // Dense kernels only: A [G][pk_rows(M) x K] and W^T [G][pk_rows(N) x K] in the packed
  // operand layout; EPI_GELU then writes C packed ([G][pk_rows(M) x N]) and EPI_RESID reads
  // R packed, C stays row-major.  Strides are ignored.  GEMM_PACKED_W: only W^T is packed, A,
  // C, R and U are contiguous row-major (EPI_GELU_SAVE, EPI_RESID; gemm_packed_w_supported).
  int packed;
  // Dense kernels only, operands stored transposed (the backward products):
  //   at: A is [G][K][M], element (m, k) at A + g * sa + k * lda + m (lda = 0: M, sa = 0: K * M)
  //   bt: W is [G][N][K], element (k, n) at W + g * N * K + n * K + k
  int at, bt;
  void* U;         // EPI_GELU_SAVE: GELU' at the pre-activations
  const void* A_scale;  // MXFP8 products: scales of A, of W (per group [pk_rows x K / 32]),
  const void* W_scale;  // and of C (EPI_GELU_MX)
  void* C_scale;
  float* colsum;   // EPI_GELU_BWD, EPI_RESID32: per-wave column sums, nullable
};
// Rows of the per-wave column sums of one group: two per 256-row tile.
__host__ __device__ inline int colsum_rows(int M) { return 2 * ((M + 255) / 256); }
// Rows per token up to which the dense launch uses 64-row tiles (measured at the 1B shapes:
// at 128 rows they run GEMM1 15 % faster than one 256-row tile and GEMM2 as fast; from 256
// rows on the 256-row tiles win).
constexpr int GEMM_SMALL_M = 128;

// True when the bf16 MFMA kernel handles this shape (else the generic kernel runs);
// lda = 0 means K (M with at).
bool gemm_uses_mfma(int dtype, int M, int N, int K, int64_t lda = 0, int at = 0, int bt = 0);
// Sparse-MoE grouped GEMM launch (bf16 MFMA only); `max_rows` bounds every group's rows.
hipError_t launch_gemm_moe(int epi, const GemmArgs& a, hipStream_t stream);
// packed: W is the groups' W^T in the packed operand layout (256 x 384 tiles, N % 384 == 0).
bool gemm_moe_supported(int N, int K, int64_t a_rows, bool packed);
// The products of prepared W^T with row-major A (GEMM_PACKED_W): N % 384 == 0, K % 32 == 0,
// A's M x K and the packed W^T below 2^31 bytes.
bool gemm_packed_w_supported(int64_t M, int64_t N, int64_t K);
hipError_t gemm_init();
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t stream);
// True when launch_gemm(dtype, epi, a) runs a matrix-core kernel that writes a.colsum.
bool gemm_writes_colsum(int dtype, int epi, const GemmArgs& a);
// MXFP8 products on the matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4): A [G][pk_rows(M)
// x K] and W^T [G][pk_rows(N) x K] in the MXFP8 layout (codes in A / W, scales in A_scale /
// W_scale); K % 64 == 0, N % 32 == 0; epi EPI_GELU_MX or EPI_RESID.
bool gemm_mx_supported(int M, int N, int K);
hipError_t launch_gemm_mx(int epi, const GemmArgs& a, hipStream_t stream);
// W [G][K][N] (bf16, row-major) -> W^T [G][pk_rows(N) x K] in MXFP8 (codes to `codes`,
// scales to `scales`, padding rows zero); K % 64 == 0.
hipError_t launch_pack_weights_mx(const void* W, void* codes, void* scales, int G, int K, int N,
                                  hipStream_t stream);
// W [G][K][N] (bf16, row-major) -> W^T [G][pk_rows(N) x K] in the packed operand layout
// (padding rows zero); K % 32 == 0.
hipError_t launch_pack_weights(const void* W, void* out, int G, int K, int N, hipStream_t stream);

}  // namespace rmx
