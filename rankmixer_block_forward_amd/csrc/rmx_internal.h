// Host-side interface between the C ABI layer (rmx_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---------------------------------------------------------------- grouped GEMM
// G independent products C_g = A_g W_g (+ epilogue), g = 0..G-1 (one per token):
//   A [G, M, K] (dtype)   W [G, K, N] (dtype)   bias [G, N] (dtype, nullable)
//   EPI_GELU:  C [G, M, N] (dtype) = GELU(A W + bias)
//   EPI_RESID: C [G, M, N] (fp32)  = A W + bias + R,  R [G, M, N] (dtype)
enum Epilogue { EPI_GELU = 0, EPI_RESID = 1 };

struct GemmArgs {
  const void* A;
  const void* W;
  const void* bias;
  const void* R;
  void* C;
  int G, M, N, K;
};

// True when the bf16 MFMA kernel handles this shape (else the generic kernel runs).
bool gemm_uses_mfma(int dtype, int M, int N, int K);
hipError_t gemm_init();
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t stream);

}  // namespace rmx
