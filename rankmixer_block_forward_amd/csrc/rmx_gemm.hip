// Grouped GEMMs of the per-token FFN: token t multiplies its rows S[t] (or the hidden
// activations) by its own weights, all T products in one launch.
// RankMixer paper translation, section 3.3.2 eq (6)-(9) (per-token FFN) and section
// 4.6 (the parallel per-token FFNs fused into one operator); "RankMixer 详解（1）",
// section 4.3 (the batch rows share each token's weights).
//
// Two kernels:
//   gemm_bf16_mfma  bf16 inputs, fp32 accumulation on the CDNA4 matrix cores
//                   (v_mfma_f32_32x32x16_bf16).  Needs K % 32 == 0 and N % 8 == 0;
//                   any M (rows past M are zero-filled and never stored).
//   gemm_generic    any shape, fp32 or bf16 inputs, fp32 FMA on the vector ALUs
//                   (the fp32 path and shapes the MFMA kernel does not take).
// Epilogues: EPI_GELU writes GELU(acc + bias) in the input dtype (the hidden
// activations); EPI_RESID writes acc + bias + R in fp32 (the pre-LN2 rows).
#include <cstdlib>
#include <cstring>

#include "rmx_device.h"
#include "rmx_internal.h"

namespace rmx {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ MFMA kernel
// Workgroup tile 256 x 256, 4 waves in a 2 x 2 grid, each wave 128 x 128 as 4 x 4 blocks
// of 32 x 32 MFMA accumulators (256 fp32 accumulator registers per lane, 1 wave per SIMD).
//
// Operand staging: K steps of 32 stream through a ring of NS = 4 LDS stages (32 KB each:
// A 256 x 32 and W 32 x 256, both as they lie in memory).  Global -> LDS copies are
// buffer loads with the LDS destination (no VGPR round trip, no LDS store instructions);
// each wave issues 8 of 16 bytes per lane per K step, K step i+4 issued while step i is
// consumed, so each load has three steps of compute to arrive.  A fragments are plain
// 16-byte LDS reads; W fragments come out of the [k][n] tile already transposed through
// the gfx950 transposing LDS read (ds_read_b64_tr_b16, two per 32 x 32 block).
// 16-byte chunks are XOR-swizzled per row so that both fragment reads are free of bank
// conflicts for 32- and 64-bank LDS models; the copy-in applies the same swizzle through
// its per-lane source address.
//
// The copies are issued from inline assembly on purpose: the compiler cannot tell which
// ring stage an LDS-destination load writes, and for a builtin it waits for every such
// load before any transposing read, which would serialize the ring.  All waits on the
// copies are therefore explicit: a wave waits for its own copies of the next stage, then
// the workgroup barrier publishes them.  Buffer loads return zero outside the token's
// slice, so ragged M and N need no branches; rows >= M and columns >= N of the tile are
// computed on zeros and never stored.
constexpr int BM = 256, BN = 256, BK = 32, NS = 4;
constexpr int A_STAGE_BYTES = BM * BK * 2;                 // 16 KB, rows of 64 B
constexpr int STAGE_BYTES = A_STAGE_BYTES + BK * BN * 2;   // + 16 KB, rows of 512 B
constexpr int MFMA_THREADS = 256;


// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Chunk swizzles.  A rows hold 4 chunks (64 B): 16 consecutive rows read one chunk each.
// W rows hold 32 chunks (512 B): a transposing read takes 4 consecutive k rows x 32 B.
__device__ __forceinline__ int swz_a(int m) { return ((m >> 1) ^ (m >> 2)) & 3; }
__device__ __forceinline__ int swz_w(int k) { return (0x0C0A0600u >> (8 * (k & 3))) & 0xff; }

struct Frags {
  u32x4_t a[4];  // A rows of the 4 row blocks: 8 bf16 each
  u32x2_t b[8];  // W columns of the 4 column blocks: k 0..3 and 4..7, 4 bf16 each
};

// MFMA 32x32x16 operand layout: lane l supplies row (l % 32) of the first operand and
// column (l % 32) of the second, each with the 8 consecutive k at 8 (l / 32) of the 16-k
// sub-step; lane l, register r of the result holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.  The W fragment goes first, so each block holds the transposed product:
// lane l owns output row l % 32 of the block and, in registers 4 g .. 4 g + 3, the four
// consecutive output columns 8 g + 4 (l / 32) .. + 3.
__device__ __forceinline__ void mfma_block(f32x16_t (&acc)[4][4], const Frags& f, int i, int j) {
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, f.a[i]);
  u32x2_t both[2] = {f.b[2 * j], f.b[2 * j + 1]};
  const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(both);
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[i][j], 0, 0, 0);
}

// Buffer descriptor over [base, base + bytes), built from wave-uniform values so that it
// lives in scalar registers (the copies below take it as an SGPR operand).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0,
                                           int(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}

// One LDS-destination buffer load: 64 lanes x 16 B to lds_dst + 16 * lane.
__device__ __forceinline__ void copy_to_lds(uint32_t lds_dst, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc,
                                            int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// One 256 x 256 output tile: the operand sources of its K loop.
struct TileSrc {
  __amdgpu_buffer_rsrc_t rA, rW;
  uint32_t offA[4], offW[4];  // per-lane byte offsets of this lane's copies (K step 0)
  uint32_t stepA, stepW;      // transposed A: bytes per K step added to every copy offset
};

// Per-lane copy offsets.  Copy-in: wave w fills A rows 64w .. 64w+63 (4 loads of 16 rows)
// and W k-rows 8w .. 8w+7 (4 loads of 2 rows) of a stage; lane q lands in LDS chunk q of
// its load, so the swizzle is applied by choosing the chunk each lane fetches.  `a_row`
// maps a tile row to the byte offset of its first element in A, or `a_oob` when the row
// does not exist (the buffer load then returns zeros).
template <typename RowOff>
__device__ __forceinline__ void tile_offsets(TileSrc& ts, int wave, int lane, int n0, int N, RowOff a_row,
                                             uint32_t bytesW) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = 64 * wave + 16 * a + (lane >> 2);
    const int c = (lane & 3) ^ swz_a(r);
    ts.offA[a] = a_row(r, c * 16);
    const int kr = 8 * wave + 2 * a + (lane >> 5);
    const int col = n0 + (((lane & 31) ^ swz_w(kr)) * 8);
    ts.offW[a] = col < N ? (uint32_t(kr) * uint32_t(N) + uint32_t(col)) * 2u : bytesW;
  }
}

// Operands stored the other way round (the backward products):
//   AT: A is [K][M] (M contiguous, k rows lda apart): its stage holds 32 k rows x 256 m,
//       laid out, copied and read like the W tile (transposing fragment reads).  The K
//       step is folded into each lane's offset (stepA), so that k rows past K fall outside
//       the buffer range and load zeros: any K works.
//   BT: W is [N][K] (K contiguous): its stage holds 256 n rows x 32 k, laid out, copied and
//       read like the A tile (plain fragment reads); K % 32 == 0.
// With AT the W tile (not transposed) also takes its K step through the lane offsets.
template <bool AT, bool BT>
__device__ __forceinline__ void tile_offsets_t(TileSrc& ts, int wave, int lane, int m0, int n0, int M, int N,
                                               int K, uint32_t lda, uint32_t bytesA, uint32_t bytesW) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (AT) {
      const int kr = 8 * wave + 2 * a + (lane >> 5);
      const int m = m0 + (((lane & 31) ^ swz_w(kr)) * 8);
      ts.offA[a] = m < M ? (uint32_t(kr) * lda + uint32_t(m)) * 2u : bytesA;
    } else {
      const int r = 64 * wave + 16 * a + (lane >> 2);
      const int c = (lane & 3) ^ swz_a(r);
      ts.offA[a] = m0 + r < M ? (uint32_t(m0 + r) * lda + uint32_t(c * 8)) * 2u : bytesA;
    }
    if constexpr (BT) {
      const int r = 64 * wave + 16 * a + (lane >> 2);
      const int c = (lane & 3) ^ swz_a(r);
      ts.offW[a] = n0 + r < N ? (uint32_t(n0 + r) * uint32_t(K) + uint32_t(c * 8)) * 2u : bytesW;
    } else {
      const int kr = 8 * wave + 2 * a + (lane >> 5);
      const int col = n0 + (((lane & 31) ^ swz_w(kr)) * 8);
      ts.offW[a] = col < N ? (uint32_t(kr) * uint32_t(N) + uint32_t(col)) * 2u : bytesW;
    }
  }
  ts.stepA = uint32_t(BK) * lda * 2u;
  ts.stepW = uint32_t(BK) * uint32_t(N) * 2u;
}

// The K loop of one tile: acc (zeroed here) += A_tile (256 x K) * W_tile (K x 256).
// Ends with every copy drained and the workgroup synchronized, so that the ring memory
// can be reused by the caller.  AT / BT: operands stored transposed (tile_offsets_t).
template <bool AT = false, bool BT = false>
__device__ __forceinline__ void mfma_tile(f32x16_t (&acc)[4][4], const TileSrc& ts, lds_u8* smem, uint32_t lds0,
                                          int K, int N, int wave, int lane) {
  const int nk = AT ? (K + BK - 1) / BK : K / BK;
  // Copy q (0..7) of K step kt into ring stage `stage`; steps past the end reload the last
  // step (in bounds, never read) so that every K step issues the same number of loads.
  auto copy = [&](int kt, int stage, int q) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * STAGE_BYTES;
    if (q < 4) {
      if constexpr (AT) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + uint32_t(8 * wave + 2 * q) * 512u);
        copy_to_lds(dst, ts.offA[q] + uint32_t(kt) * ts.stepA, ts.rA, 0);
      } else {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + uint32_t(64 * wave + 16 * q) * 64u);
        copy_to_lds(dst, ts.offA[q], ts.rA, kt * BK * 2);
      }
    } else if constexpr (BT) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(sbase + A_STAGE_BYTES + uint32_t(64 * wave + 16 * (q - 4)) * 64u);
      copy_to_lds(dst, ts.offW[q - 4], ts.rW, kt * BK * 2);
    } else {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(sbase + A_STAGE_BYTES + uint32_t(8 * wave + 2 * (q - 4)) * 512u);
      if constexpr (AT)
        copy_to_lds(dst, ts.offW[q - 4] + uint32_t(kt) * ts.stepW, ts.rW, 0);
      else
        copy_to_lds(dst, ts.offW[q - 4], ts.rW, kt * BK * N * 2);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  // Per-lane byte offsets of this wave's fragments within a stage.  Row-tile fragments
  // (A, or W with BT) are plain 16-byte reads per K sub-step; k-row-tile fragments (W, or
  // A with AT) are two transposing reads per K sub-step.
  // transposing read: lane l of each 16-lane group addresses k row kb + (l % 16) / 4 and
  // 4 consecutive columns at 4 (l % 4); it receives column (l % 16) of that 4 x 16 block
  const int kb = 8 * (lane >> 5) + ((lane & 15) >> 2);
  auto row_frag_off = [&](int base, int m, int kk) {
    const int c = kk * 2 + (lane >> 5);
    return uint32_t(base + m * 64 + ((c ^ swz_a(m)) << 4));
  };
  auto tr_frag_off = [&](int base, int n) {
    return uint32_t(base + kb * 512 + (((n >> 3) ^ swz_w(kb)) << 4) + (n & 7) * 2);
  };
  uint32_t aoff[2][4], boff[4];  // row-tile A per sub-step; k-row-tile W (sub-step 1 at + 16 rows)
  uint32_t aoff_t[4], boff_r[2][4];  // AT: k-row-tile A; BT: row-tile W
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (AT) {
      aoff_t[i] = tr_frag_off(0, wm * 128 + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) aoff[kk][i] = row_frag_off(0, wm * 128 + i * 32 + (lane & 31), kk);
    }
    if constexpr (BT) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) boff_r[kk][i] = row_frag_off(A_STAGE_BYTES, wn * 128 + i * 32 + (lane & 31), kk);
    } else {
      boff[i] = tr_frag_off(A_STAGE_BYTES, wn * 128 + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    }
  }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  auto tr_read = [](const lds_u8* q) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q));
  };
  auto read_frags = [&](Frags& f, const lds_u8* stage_ptr, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (AT) {
        const lds_u8* q = stage_ptr + aoff_t[i] + kk * 16 * 512;
        const u32x2_t lo = tr_read(q), hi = tr_read(q + 4 * 512);
        f.a[i] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      } else {
        f.a[i] = *reinterpret_cast<const lds_u32x4*>(stage_ptr + aoff[kk][i]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BT) {
        const u32x4_t v = *reinterpret_cast<const lds_u32x4*>(stage_ptr + boff_r[kk][j]);
        f.b[2 * j] = u32x2_t{v.x, v.y};
        f.b[2 * j + 1] = u32x2_t{v.z, v.w};
      } else {
        const lds_u8* q = stage_ptr + boff[j] + kk * 16 * 512;
        f.b[2 * j] = tr_read(q);
        f.b[2 * j + 1] = tr_read(q + 4 * 512);
      }
    }
  };

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Prologue: K steps 0..NS-1 into the NS stages; wait for step 0 (8 loads per step).
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int q = 0; q < 8; ++q) copy(s, s, q);
  asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
  Frags f0, f1;
  read_frags(f0, smem, 0);

  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * STAGE_BYTES;
    const int nstage = stage + 1 == NS ? 0 : stage + 1;
    // sub-step 0: MFMAs on f0 while the fragments of sub-step 1 are read
    read_frags(f1, sp, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_block(acc, f0, i, j);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
    // Every read of this stage has returned (f1 included) before the barrier; after it,
    // step it+1 is visible (each wave waited for its own copies: 16 later loads may be
    // outstanding) and this stage may be refilled with step it+NS.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1: MFMAs on f1, the copies of step it+NS spread between them, and the first
    // fragments of the next stage read
    read_frags(f0, smem + nstage * STAGE_BYTES, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mfma_block(acc, f1, q >> 1, (q & 1) * 2);
      mfma_block(acc, f1, q >> 1, (q & 1) * 2 + 1);
      __builtin_amdgcn_sched_barrier(0);
      copy(it + NS, stage, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  // Drain the trailing copies before the ring memory is reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Epilogue of one tile: the wave's NI x NJ blocks of 32 x 32, whose top-left element is
// tile row wrow0, tile column wcol0 (n0 + wcol0 in the output).  Accumulator layout of a
// block (transposed product): lane l holds row l % 32 and, in register 4 g + e, column
// 8 g + 4 (l / 32) + e.  Each wave stages 32 rows x 32 NJ columns at a time through LDS
// (16-byte writes) so that every lane then owns 8 consecutive columns of one row: 16-byte
// global stores, and coalesced bias / residual loads.  `row_of(m)` is the output row (in
// group g) of tile row m, or -1 if the row does not exist; C (and R) rows are p.ldc apart
// and groups p.sc apart, except that with PK the GELU output and the residual are in the
// packed operand layout.
template <int EPI, int NI, int NJ, bool PK, typename RowOf>
__device__ __forceinline__ void tile_epilogue(const f32x16_t (&acc)[NI][NJ], float* smem_f, const GemmArgs& p,
                                              const bf16_t* bias_g, int n0, int wrow0, int wcol0, int wave,
                                              int lane, int g, RowOf row_of, int colsum_row = 0) {
  constexpr int LD = NJ * 32 + 4;     // fp32 row stride of the staging rows
  constexpr int LPR = NJ * 4;         // lanes per staged row (8 columns each)
  constexpr int RPP = 64 / LPR;       // rows per pass
  const int N = p.N;
  float* st = smem_f + wave * 32 * LD;
  const int col8 = (lane % LPR) * 8;
  const int rsub = lane / LPR;
  const int n = n0 + wcol0 + col8;
  const bool n_ok = n < N;
  float bias[8], csum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bias[e] = csum[e] = 0.f;
  if (bias_g && n_ok) load8(bias_g + n, bias);

#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 v = make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                                     acc[i][j][4 * g4 + 3]);
        *reinterpret_cast<float4*>(st + (lane & 31) * LD + j * 32 + 8 * g4 + 4 * (lane >> 5)) = v;
      }
    // the staging rows are private to this wave, whose LDS operations complete in order
    asm volatile("" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int row = pass * RPP + rsub;
      const int orow = row_of(wrow0 + i * 32 + row);
      float v[8];
      const float4 x0 = *reinterpret_cast<const float4*>(st + row * LD + col8);
      const float4 x1 = *reinterpret_cast<const float4*>(st + row * LD + col8 + 4);
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
      v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      if constexpr (EPI == EPI_GELU_MX) {
        // GELU, then MXFP8 along the row: the 32 columns of one scale block are the 8
        // columns of 4 neighbouring lanes of this row (the exchange runs on every lane)
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = gelu_erf(v[e] + bias[e]);
          amax = fmaxf(amax, fabsf(v[e]));
        }
        amax = quad_max(amax);
        const uint32_t sb = mx_scale_bits(amax);
        const float inv = mx_inv_scale(sb);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= inv;
        const uint2 q = e4m3_pack8(v);
        if (orow >= 0 && n_ok) {
          const size_t gm = size_t(g) * size_t(pk_rows(p.M)) * size_t(N);
          *reinterpret_cast<uint2*>(static_cast<uint8_t*>(p.C) + gm + mx_off(orow, n, N) + ((n >> 3) & 1) * 8) = q;
          if ((lane & 3) == 0) static_cast<uint8_t*>(p.C_scale)[gm / 32 + mx_scale_off(orow, n >> 5, N)] = uint8_t(sb);
        }
        continue;
      }
      if (orow >= 0 && n_ok) {
        const size_t off = size_t(g) * size_t(p.sc) + size_t(orow) * size_t(p.ldc) + n;
        size_t pko = 0;
        if constexpr (PK) pko = size_t(g) * size_t(pk_rows(p.M)) * N + pk_off(orow, n, N);
        if constexpr (EPI == EPI_GELU || EPI == EPI_MOE1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[e]);
          store8(static_cast<bf16_t*>(p.C) + (PK ? pko : off), v);
        } else if constexpr (EPI == EPI_GELU_SAVE) {
          float gd[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_erf_and_grad(v[e] + bias[e], &gd[e]);
          store8(static_cast<bf16_t*>(p.U) + off, gd);
          store8(static_cast<bf16_t*>(p.C) + off, v);
        } else if constexpr (EPI == EPI_GELU_BWD) {
          float gd[8];
          load8(static_cast<const bf16_t*>(p.R) + off, gd);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] *= gd[e];
            csum[e] += v[e];
          }
          store8(static_cast<bf16_t*>(p.C) + off, v);
        } else if constexpr (EPI == EPI_RESID32) {
          float rr[8];
          load8(static_cast<const float*>(p.R) + off, rr);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] += rr[e];
            csum[e] += rr[e];
          }
          store8(static_cast<float*>(p.C) + off, v);
        } else if constexpr (EPI == EPI_STORE32) {
          store8(static_cast<float*>(p.C) + off, v);
        } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += bias[e];
          store8(static_cast<bf16_t*>(p.C) + off, v);
        } else if constexpr (EPI == EPI_RESID) {
          float rr[8];
          load8(static_cast<const bf16_t*>(p.R) + (PK ? pko : off), rr);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] + bias[e] + rr[e];
          store8(static_cast<float*>(p.C) + off, v);
        } else {
          const float gv = p.row_gate[orow];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gv * (v[e] + bias[e]);
          store8(static_cast<bf16_t*>(p.C) + off, v);
        }
      }
    }
    asm volatile("" ::: "memory");
  }
  if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_RESID32) {
    // column sums over the wave's rows: lanes that share columns meet by butterfly exchange
    if (p.colsum) {
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) csum[e] += __shfl_xor(csum[e], off, 64);
      if (rsub == 0 && n_ok)
        store8(p.colsum + (size_t(g) * colsum_rows(p.M) + colsum_row) * N + n, csum);
    }
  }
  // every wave is done with its staging rows before the ring memory is reused
  __syncthreads();
}

// K loop of one 256 x 256 tile over packed operands: K steps of 32 through a 3-stage ring;
// a stage is the tile's 16 KB A block and 16 KB W^T block of that step, each copied as 16
// contiguous 1 KB pieces (4 per wave); both fragments are plain 16-byte LDS reads.
constexpr int PK_NS = 3;
__device__ __forceinline__ void mfma_tile_pk(f32x16_t (&acc)[4][4], __amdgpu_buffer_rsrc_t rA,
                                             __amdgpu_buffer_rsrc_t rW, lds_u8* smem, uint32_t lds0, int K,
                                             int wave, int lane) {
  const int nk = K / BK;
  auto copy = [&](int kt, int stage, int q) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * STAGE_BYTES;
    const uint32_t piece = uint32_t(4 * wave + (q & 3));
    const uint32_t voff = piece * 1024u + uint32_t(lane) * 16u;
    if (q < 4) copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), voff, rA, kt * 16384);
    else copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + A_STAGE_BYTES + piece * 1024u), voff, rW, kt * 16384);
  };
  const int wm = wave >> 1, wn = wave & 1;
  uint32_t aoff[2][4], boff[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = kk * 2 + (lane >> 5);
      const int m = wm * 128 + i * 32 + (lane & 31);
      aoff[kk][i] = pk_lds_off(m, c);
      const int n = wn * 128 + i * 32 + (lane & 31);
      boff[kk][i] = uint32_t(A_STAGE_BYTES) + pk_lds_off(n, c);
    }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  struct PkFrags {
    u32x4_t a[4];  // A rows of the 4 row blocks: 8 bf16 each
    u32x4_t b[4];  // W^T rows (output columns) of the 4 column blocks: 8 bf16 each
  };
  auto read_frags = [&](PkFrags& f, const lds_u8* sp, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[kk][i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const lds_u32x4*>(sp + boff[kk][j]);
  };
  auto mm = [&](const PkFrags& f, int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.b[j]),
                                                        __builtin_bit_cast(bf16x8_t, f.a[i]), acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // prologue: steps 0..PK_NS-1; wait for step 0 (8 loads per step)
#pragma unroll
  for (int st = 0; st < PK_NS; ++st)
#pragma unroll
    for (int q = 0; q < 8; ++q) copy(st, st, q);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  PkFrags f0, f1;
  read_frags(f0, smem, 0);
  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * STAGE_BYTES;
    const int nstage = stage + 1 == PK_NS ? 0 : stage + 1;
    read_frags(f1, sp, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mm(f0, i, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8, 0);
    // every read of this stage has returned; after the barrier step it+1 is visible (the 8
    // loads of the step after it may be outstanding) and this stage takes step it+PK_NS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f0, smem + nstage * STAGE_BYTES, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mm(f1, q >> 1, (q & 1) * 2);
      mm(f1, q >> 1, (q & 1) * 2 + 1);
      __builtin_amdgcn_sched_barrier(0);
      copy(it + PK_NS, stage, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Dense per-token GEMM: one workgroup per tile, G * ceil(M/256) * ceil(N/256) tiles; PK:
// operands in the packed layout.
template <int EPI, bool PK, bool AT = false, bool BT = false>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_mfma(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[NS * STAGE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;  // the generic pointer of a __shared__ array is in LDS
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = (N + BN - 1) / BN;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  // Within a token, tiles run over bands of TILE_BAND row tiles: M-fastest inside a band,
  // then N, then the next band, so the tiles resident on one XCD at a time form a compact
  // block whatever the batch size.
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;

  f32x16_t acc[4][4];
  if constexpr (PK) {
    // the tile's A blocks (row block mt) and W^T blocks (row block nt): K/32 x 16 KB each
    const uint32_t blk = uint32_t(K / BK) * 16384u;
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(static_cast<const uint16_t*>(p.A) + (size_t(g) * nMt + mt) * (size_t(blk) / 2), blk);
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(static_cast<const uint16_t*>(p.W) + (size_t(g) * nNt + nt) * (size_t(blk) / 2), blk);
    mfma_tile_pk(acc, rA, rW, smem, lds0, K, wave, lane);
  } else if constexpr (AT || BT) {
    // Slices are < 2^31 bytes (checked at launch).
    const uint32_t lda = uint32_t(p.lda);
    const uint32_t bytesA = AT ? uint32_t(K) * lda * 2u : (uint32_t(M - 1) * lda + uint32_t(K)) * 2u;
    const uint32_t bytesW = uint32_t(K) * uint32_t(N) * 2u;
    TileSrc ts;
    ts.rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(g) * size_t(p.sa), bytesA);
    ts.rW = make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * K * N, bytesW);
    tile_offsets_t<AT, BT>(ts, wave, lane, m0, n0, M, N, K, lda, bytesA, bytesW);
    mfma_tile<AT, BT>(acc, ts, smem, lds0, K, N, wave, lane);
  } else {
    // Slices are < 2^31 bytes (checked at launch); an offset equal to the slice size is out
    // of range whether or not the uniform offset takes part in the range check.
    const uint32_t lda = uint32_t(p.lda);
    const uint32_t bytesA = (uint32_t(M - 1) * lda + uint32_t(K)) * 2u, bytesW = uint32_t(K) * uint32_t(N) * 2u;
    TileSrc ts;
    ts.rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(g) * size_t(p.sa), bytesA);
    ts.rW = make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * K * N, bytesW);
    tile_offsets(ts, wave, lane, n0, N,
                 [&](int r, int cbytes) {
                   return (m0 + r < M) ? uint32_t(m0 + r) * lda * 2u + uint32_t(cbytes) : bytesA;
                 },
                 bytesW);
    mfma_tile(acc, ts, smem, lds0, K, N, wave, lane);
  }
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue<EPI, 4, 4, PK>(acc, reinterpret_cast<float*>(smem_g), p, bias_g, n0, (wave >> 1) * 128,
                               (wave & 1) * 128, wave, lane, g, [&](int m) { return m0 + m < M ? m0 + m : -1; },
                               2 * mt + (wave >> 1));
}

// ------------------------------------------------------- 256 x 384 and 128 x 384 tiles
// Where N is a multiple of 384, the packed-operand products run 256 x 384 tiles: each wave
// owns 128 x 192 outputs (4 x 6 blocks of 32 x 32), and the operand bytes copied into LDS per
// FLOP drop by 17 % against 256 x 256 tiles (the copy rate of a CU bounds the K loop).  The
// 384 accumulators per lane exceed the 256 AGPRs: column blocks 0..3 use the builtin (the
// compiler keeps them in AGPRs), blocks 4..5 an MFMA in inline assembly with VGPR
// accumulators.  The compiler does not see the instruction inside the assembly, so explicit
// wait states guard its VGPR hazards: after the VALU zeroes the accumulators, before a
// fragment register an assembly MFMA has read is rewritten by an LDS read, and before the
// epilogue reads the results.  Per block, the products are accumulated in the same order as
// in the 256 x 256 kernel, so the two give the same bits.  The same K loop and epilogue
// also run 128 x 384 tiles (waves of 64 x 192; see mfma_tile_pk6).
constexpr int BN6 = 384;
constexpr int STAGE6_BYTES = A_STAGE_BYTES + BN6 * BK * 2;  // 16 KB of A + 24 KB of W^T
constexpr int PK6_NS = 3;
constexpr int LD6 = 2 * 32 + 4;                             // epilogue staging rows: 64 columns

// K loop of one 256 x 384 tile.  A stage holds the tile's 16 KB A block and three 8 KB halves
// (128 output columns each) of W^T blocks: 40 contiguous 1 KB pieces, 10 per wave (wave w
// takes pieces w, w + 4, ...: 4 of A and 6 of W^T).  W^T half-block H = 3 nt + (piece / 8)
// of the token is rows 128 H .. 128 H + 127: block H / 2, half H % 2.  Row r of the stage's
// W^T part is tile column r; the chunk swizzle depends on r % 8, which a half-block keeps.
// GATHER_A: A is not packed but gathered from row-major rows; offA[c] is this lane's byte
// offset of piece wave + 4 c at K step 0 (the 16 bytes that belong at the lane's place in
// the packed layout), and a K step advances it by 64 bytes.  NI < TM / 64: only the wave's
// first NI row blocks hold rows (a tile past the end of its rows); the others are neither
// read nor multiplied and their accumulators stay zero.  Copies and barriers are the same
// for every NI, so the waves of one workgroup may run different NI.
// TM = 128: tiles of 128 x 384 (waves of 64 x 192, 2 x 6 blocks) for launches that would
// leave CUs idle with 256-row tiles; the A part of a stage is then 8 KB (the first or second
// half of a packed 256-row block, selected by the caller's rA) and a wave copies 8 pieces
// per K step instead of 10.  The sums run in the same order for every TM.
template <bool GATHER_A, int NI, int TM = 256>
__device__ __forceinline__ void mfma_tile_pk6(f32x16_t (&accA)[4][4], f32x16_t (&accV)[4][2],
                                              __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rW, lds_u8* smem,
                                              uint32_t lds0, int K, int nt, int wave, int lane,
                                              const uint32_t (&offA)[4]) {
  static_assert(TM == 256 || TM == 128, "256- or 128-row tiles");
  static_assert(!GATHER_A || TM == 256, "gathered rows use 256-row tiles");
  static_assert(NI <= TM / 64, "row blocks of a wave");
  constexpr int APW = TM / 64;                 // A pieces per wave and K step
  constexpr int NCP = APW + 6;                 // copies per wave and K step
  constexpr int ABYTES = TM * BK * 2;          // A part of a stage
  constexpr int STG = ABYTES + BN6 * BK * 2;   // stage bytes
  const int nk = K / BK;
  uint32_t voffW[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const int q = wave + 4 * c;
    const int hb = 3 * nt + (q >> 3);
    voffW[c] = uint32_t(hb >> 1) * uint32_t(nk) * 16384u + uint32_t(hb & 1) * 8192u + uint32_t(q & 7) * 1024u +
               uint32_t(lane) * 16u;
  }
  // copy c (0..NCP-1) of K step kt into ring stage `stage`; steps past the end reload the
  // last step (in bounds, never read) so that every K step issues the same number of loads
  auto copy = [&](int kt, int stage, int c) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * STG;
    if (c < APW) {
      const uint32_t piece = uint32_t(wave + 4 * c);
      if constexpr (GATHER_A)
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), offA[c], rA, kt * BK * 2);
      else
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), piece * 1024u + uint32_t(lane) * 16u, rA,
                    kt * 16384);
    } else {
      const uint32_t q = uint32_t(wave + 4 * (c - APW));
      copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + ABYTES + q * 1024u), voffW[c - APW], rW, kt * 16384);
    }
  };
  const int wm = wave >> 1, wn = wave & 1;
  uint32_t aoff[2], boff[2];  // row block i / column block j at + 2048 i / + 2048 j
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = kk * 2 + (lane >> 5);
    const int m = wm * (TM / 2) + (lane & 31);
    aoff[kk] = pk_lds_off(m, c);
    const int n = wn * 192 + (lane & 31);
    boff[kk] = uint32_t(ABYTES) + pk_lds_off(n, c);
  }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  // a0 / a1: A fragments of sub-steps 0 / 1; b[j]: the W^T fragment of column block j,
  // refilled right after the MFMAs that use it (sub-step 1 of this stage, then sub-step 0 of
  // the next), which keeps the fragments at 56 registers
  u32x4_t a0[4], a1[4], b[6];
  auto read_a = [&](u32x4_t (&a)[4], const lds_u8* sp, int kk) {
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[kk] + i * 2048);
  };
  auto read_b = [&](const lds_u8* sp, int kk, int j) {
    if (j >= 4) asm volatile("s_nop 7" ::: "memory");  // an assembly MFMA read b[j] just before
    b[j] = *reinterpret_cast<const lds_u32x4*>(sp + boff[kk] + j * 2048);
  };
  auto mm = [&](const u32x4_t (&a)[4], int i, int j) {
    if (i >= NI) return;
    if (j < 4)
      accA[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                           __builtin_bit_cast(bf16x8_t, a[i]), accA[i][j], 0, 0, 0);
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(accV[i][j - 4]) : "v"(b[j]), "v"(a[i]));
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) accA[i][j][r] = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) accV[i][j][r] = 0.f;
  }
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // the zeroed VGPR accumulators settle
  // prologue: steps 0..PK6_NS-1; wait for step 0 (NCP loads per step)
#pragma unroll
  for (int st = 0; st < PK6_NS; ++st)
#pragma unroll
    for (int c = 0; c < NCP; ++c) copy(st, st, c);
  if constexpr (NCP == 10)
    asm volatile("s_waitcnt vmcnt(20)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  read_a(a0, smem, 0);
#pragma unroll
  for (int j = 0; j < 6; ++j) read_b(smem, 0, j);
  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * STG;
    const int nstage = stage + 1 == PK6_NS ? 0 : stage + 1;
    // sub-step 0 on a0 / b; sub-step 1's fragments of this stage read behind the MFMAs
    read_a(a1, sp, 1);
#pragma unroll
    for (int j = 0; j < 6; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mm(a0, i, j);
      __builtin_amdgcn_sched_barrier(0);
      read_b(sp, 1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every read of this stage has returned; after the barrier step it+1 is visible (the NCP
    // loads of the step after it may be outstanding) and this stage takes step it+PK6_NS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NCP == 10)
      asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1 on a1 / b; the next stage's sub-step 0 fragments and this stage's refill
    // between the MFMAs
    const lds_u8* np = smem + nstage * STG;
    read_a(a0, np, 0);
#pragma unroll
    for (int j = 0; j < 6; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        mm(a1, 2 * h, j);
        mm(a1, 2 * h + 1, j);
        if (2 * j + h < NCP) {
          __builtin_amdgcn_sched_barrier(0);
          copy(it + PK6_NS, stage, 2 * j + h);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      read_b(np, 0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // the last MFMAs' results settle
  __syncthreads();
}

// Epilogue of a TM x 384 tile, the arithmetic of tile_epilogue: GELU (packed H out),
// residual (packed S in, fp32 Y out), or the Sparse-MoE ones (GELU to the compacted hidden
// rows; gate times result to the compacted output rows).  Per row block i of the wave and
// group of two column blocks, 32 rows x 64 columns are staged through LDS so that each lane
// then owns 8 consecutive columns of one row (8 lanes per row, 8 rows per pass).
// row_of(r) maps tile row r to its output row, or -1 where the tile runs past the rows.
// RM: the dense operands are row-major (the training forward): EPI_GELU_SAVE writes H and
// GELU' to C and U, EPI_RESID reads R, all [G][M][N] with the strides of p.
template <int EPI, int TM = 256, bool RM = false, typename RowOf>
__device__ __forceinline__ void tile_epilogue6(const f32x16_t (&accA)[4][4], const f32x16_t (&accV)[4][2],
                                               float* smem_f, const GemmArgs& p, int g, const bf16_t* bias_g,
                                               int n0, int wave, int lane, RowOf row_of, int nib = TM / 64) {
  const int M = p.M, N = p.N;
  const int wrow0 = (wave >> 1) * (TM / 2), wcol0 = (wave & 1) * 192;
  float* st = smem_f + wave * 32 * LD6;
  const int col8 = (lane & 7) * 8;
  float bias[3][8];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) bias[s][e] = 0.f;
    const int n = n0 + wcol0 + s * 64 + col8;
    if (bias_g && n < N) load8(bias_g + n, bias[s]);
  }
#pragma unroll
  for (int i = 0; i < TM / 64; ++i) {
    if (i >= nib) break;  // row blocks past the rows (wave-uniform)
#pragma unroll
    for (int s = 0; s < 3; ++s) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jb = 2 * s + jj;
        const f32x16_t& a = jb < 4 ? accA[i][jb] : accV[i][jb - 4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4*>(st + (lane & 31) * LD6 + jj * 32 + 8 * g4 + 4 * (lane >> 5)) =
              make_float4(a[4 * g4], a[4 * g4 + 1], a[4 * g4 + 2], a[4 * g4 + 3]);
      }
      // the staging rows are private to this wave, whose LDS operations complete in order
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int row = pass * 8 + (lane >> 3);
        const int m = row_of(wrow0 + i * 32 + row);
        const int n = n0 + wcol0 + s * 64 + col8;
        float v[8];
        const float4 x0 = *reinterpret_cast<const float4*>(st + row * LD6 + col8);
        const float4 x1 = *reinterpret_cast<const float4*>(st + row * LD6 + col8 + 4);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        if (m >= 0 && n < N) {
          const size_t rmo = size_t(g) * size_t(p.sc) + size_t(m) * size_t(p.ldc) + n;  // row-major
          if constexpr (EPI == EPI_GELU) {
            const size_t pko = size_t(g) * size_t(pk_rows(M)) * N + pk_off(m, n, N);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[s][e]);
            store8(static_cast<bf16_t*>(p.C) + pko, v);
          } else if constexpr (EPI == EPI_GELU_SAVE) {
            static_assert(RM, "the training epilogue writes row-major H and GELU'");
            float gd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf_and_grad(v[e] + bias[s][e], &gd[e]);
            store8(static_cast<bf16_t*>(p.U) + rmo, gd);
            store8(static_cast<bf16_t*>(p.C) + rmo, v);
          } else if constexpr (EPI == EPI_RESID) {
            const size_t pko = RM ? rmo : size_t(g) * size_t(pk_rows(M)) * N + pk_off(m, n, N);
            float rr[8];
            load8(static_cast<const bf16_t*>(p.R) + pko, rr);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] + bias[s][e] + rr[e];
            store8(static_cast<float*>(p.C) + rmo, v);
          } else if constexpr (EPI == EPI_MOE1) {
            // hidden rows in the packed layout, m a row of the group's tile-aligned blocks
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[s][e]);
            store8(static_cast<bf16_t*>(p.C) + pk_off(m, n, N), v);
          } else {
            const float gv = p.row_gate[m];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gv * (v[e] + bias[s][e]);
            store8(static_cast<bf16_t*>(p.C) + size_t(m) * size_t(N) + n, v);
          }
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

// Dense per-token product on packed operands with TM x 384 tiles: G * ceil(M/TM) * N/384
// workgroups, N % 384 == 0; EPI_GELU or EPI_RESID.
template <int EPI, int TM>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_mfma_n384(GemmArgs p) {
  static_assert(EPI == EPI_GELU || EPI == EPI_RESID, "TM x 384 tiles serve the inference epilogues");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[PK6_NS * (TM * BK * 2 + BN6 * BK * 2)];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + TM - 1) / TM, nNt = N / BN6;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  // bands of TILE_BAND row tiles, M-fastest inside a band (as in the 256 x 256 kernel)
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  // the tile's A blocks (packed row block, K/32 x 16 KB; a 128-row tile starts at the first or
  // second 8 KB half of each) and the token's whole W^T (pk_rows(N) rows; slices < 2^31
  // bytes, checked at launch)
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  const int nMb = (M + BM - 1) / BM;                    // packed 256-row blocks per token
  const int mb = mt / (BM / TM), half = mt % (BM / TM);  // block and half of this tile
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(static_cast<const uint16_t*>(p.A) + (size_t(g) * nMb + mb) * (size_t(blk) / 2) + size_t(half) * 4096,
                blk - uint32_t(half) * 8192u);
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
  f32x16_t accA[4][4], accV[4][2];
  const uint32_t no_gather[4] = {0u, 0u, 0u, 0u};
  mfma_tile_pk6<false, TM / 64, TM>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, no_gather);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  const int m0 = mt * TM;
  tile_epilogue6<EPI, TM>(accA, accV, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                          [&](int r) { return m0 + r < M ? m0 + r : -1; });
}

// ------------------------------------------ TM x 192 tiles (TM = 256 or 128), two per CU
// A 256 x 384 tile holds 384 fp32 accumulators per lane and fills a SIMD's registers with one
// wave, so its epilogue (bias, GELU, bf16 stores: about a quarter of the GELU product's time
// at the 1B shape) leaves the matrix cores idle.  A 256 x 192 tile needs 192 accumulators
// (AGPRs) and fits in 256 registers per lane with a 2-stage ring of 28 KB stages, so two
// workgroups share a CU and one's epilogue runs beside the other's K loop.  It copies 40 %
// more operand bytes per FLOP than the 256 x 384 tile; measured at the 1B shape, B = 2048:
// GELU product 1.17 against 1.21 ms, residual product level (1.035 against 1.03 ms), so the
// launch takes it for the GELU epilogue.  Waves 2 x 2 of (TM / 2) x 96 (TM / 64 x 3 blocks);
// per block the same MFMAs in the same K order as the other tile shapes, so the bits are the
// same.  TM = 128 (waves of 64 x 96, 3-stage ring of 20 KB stages; the A part of a stage is
// the first or second 8 KB half of a packed 256-row block) serves launches with few tiles,
// where a CU's copy rate, not the matrix cores, sets the time: it spreads a product over
// twice as many workgroups as the 128 x 384 tile.
// W^T rows of a tile: 192 nt .. 192 nt + 191, which may straddle two 256-row packed blocks;
// each 16-row piece of a stage lies inside one block (the swizzle depends on row % 8).
constexpr int BN3 = 192;
constexpr int LD3 = 32 + 4;                        // epilogue staging rows: one 32-column block

template <int TM> struct Pk3 {
  static constexpr int NI = TM / 64;               // row blocks per wave
  static constexpr int APW = TM / 64;              // A pieces per wave and K step
  static constexpr int NCP = APW + 3;              // copies per wave and K step
  static constexpr int SA = TM * BK * 2;           // A part of a stage
  static constexpr int SG = SA + BN3 * BK * 2;     // stage bytes
  static constexpr int NS = TM == 256 ? 2 : 3;     // ring stages
};

template <int TM>
__device__ __forceinline__ void mfma_tile_pk3(f32x16_t (&acc)[TM / 64][3], __amdgpu_buffer_rsrc_t rA,
                                              __amdgpu_buffer_rsrc_t rW, lds_u8* smem, uint32_t lds0, int K, int nt,
                                              int wave, int lane) {
  using C = Pk3<TM>;
  constexpr int NI = C::NI, APW = C::APW, NCP = C::NCP, SA = C::SA, SG = C::SG, NS = C::NS;
  static_assert(NCP <= 2 * 3 * NI, "the refill copies fit between the MFMAs of a sub-step");
  const int nk = K / BK;
  uint32_t voffW[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int row = BN3 * nt + 16 * (wave + 4 * c);  // first W^T row of the piece
    voffW[c] = uint32_t(row >> 8) * uint32_t(nk) * 16384u + uint32_t(row & 255) * 64u + uint32_t(lane) * 16u;
  }
  // copy c (0..NCP-1) of K step kt into stage `stage`: pieces wave + 4 c of A (c < APW) and
  // wave + 4 (c - APW) of W^T; steps past the end reload the last (in bounds, never read)
  auto copy = [&](int kt, int stage, int c) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * SG;
    if (c < APW) {
      const uint32_t piece = uint32_t(wave + 4 * c);
      copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), piece * 1024u + uint32_t(lane) * 16u, rA,
                  kt * 16384);
    } else {
      const uint32_t q = uint32_t(wave + 4 * (c - APW));
      copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + SA + q * 1024u), voffW[c - APW], rW, kt * 16384);
    }
  };
  const int wm = wave >> 1, wn = wave & 1;
  uint32_t aoff[2], boff[2];  // row block i / column block j at + 2048 i / + 2048 j
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = kk * 2 + (lane >> 5);
    const int m = wm * (TM / 2) + (lane & 31);
    aoff[kk] = pk_lds_off(m, c);
    const int n = wn * 96 + (lane & 31);
    boff[kk] = uint32_t(SA) + pk_lds_off(n, c);
  }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  u32x4_t a0[NI], a1[NI], b[3];
  auto read_a = [&](u32x4_t (&a)[NI], const lds_u8* sp, int kk) {
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[kk] + i * 2048);
  };
  auto read_b = [&](const lds_u8* sp, int kk, int j) {
    b[j] = *reinterpret_cast<const lds_u32x4*>(sp + boff[kk] + j * 2048);
  };
  auto mm = [&](const u32x4_t (&a)[NI], int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                        __builtin_bit_cast(bf16x8_t, a[i]), acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // prologue: steps 0 .. NS-1; wait for step 0 (NCP loads per step)
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int c = 0; c < NCP; ++c) copy(st, st, c);
  if constexpr (TM == 256)
    asm volatile("s_waitcnt vmcnt(7)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  read_a(a0, smem, 0);
#pragma unroll
  for (int j = 0; j < 3; ++j) read_b(smem, 0, j);
  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * SG;
    const int nstage = stage + 1 == NS ? 0 : stage + 1;
    // sub-step 0 on a0 / b; sub-step 1's fragments read behind the MFMAs that free them
    read_a(a1, sp, 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
#pragma unroll
      for (int i = 0; i < NI; ++i) mm(a0, i, j);
      __builtin_amdgcn_sched_barrier(0);
      read_b(sp, 1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every read of this stage has returned; after the barrier step it+1 is visible (with 3
    // stages the NCP loads of step it+2 may be outstanding) and this stage takes step it+NS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TM == 256)
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1 on a1 / b; the refill of this stage spread over its MFMAs
    const lds_u8* np = smem + nstage * SG;
    read_a(a0, np, 0);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        mm(a1, i, j);
        // TM = 256: copies after MFMAs 0, 2, 4, 6, 8, 9, 10 of 12; TM = 128: after 0 .. 4 of 6
        const int q = NI * j + i;
        const int c = TM == 256 ? (q <= 6 ? ((q & 1) ? -1 : q / 2) : (q <= 10 ? q - 4 : -1)) : (q < 5 ? q : -1);
        if (c >= 0) {
          __builtin_amdgcn_sched_barrier(0);
          copy(it + NS, stage, c);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      read_b(np, 0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Epilogue of a TM x 192 tile (the arithmetic of tile_epilogue6): per 32 x 32 block, the
// accumulators are staged through LDS so that each lane owns 8 consecutive columns of one row
// (4 lanes per row, 16 rows per pass).  Rows past M are not stored.
template <int EPI, int TM>
__device__ __forceinline__ void tile_epilogue3(const f32x16_t (&acc)[TM / 64][3], float* smem_f, const GemmArgs& p,
                                               int g, const bf16_t* bias_g, int n0, int m0, int wave, int lane) {
  constexpr int NI = TM / 64;
  const int M = p.M, N = p.N;
  const int wrow0 = (wave >> 1) * (TM / 2), wcol0 = (wave & 1) * 96;
  float* st = smem_f + wave * 32 * LD3;
  const int col8 = (lane & 3) * 8;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int n = n0 + wcol0 + j * 32 + col8;
    float bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bias[e] = 0.f;
    if (bias_g) load8(bias_g + n, bias);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(st + (lane & 31) * LD3 + 8 * g4 + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
      // the staging rows are private to this wave, whose LDS operations complete in order
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int row = pass * 16 + (lane >> 2);
        const int m = m0 + wrow0 + i * 32 + row;
        float v[8];
        const float4 x0 = *reinterpret_cast<const float4*>(st + row * LD3 + col8);
        const float4 x1 = *reinterpret_cast<const float4*>(st + row * LD3 + col8 + 4);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        if (m < M) {
          const size_t pko = size_t(g) * size_t(pk_rows(M)) * N + pk_off(m, n, N);
          if constexpr (EPI == EPI_GELU) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[e]);
            store8(static_cast<bf16_t*>(p.C) + pko, v);
          } else {
            float rr[8];
            load8(static_cast<const bf16_t*>(p.R) + pko, rr);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] + bias[e] + rr[e];
            store8(static_cast<float*>(p.C) + size_t(g) * size_t(p.sc) + size_t(m) * size_t(p.ldc) + n, v);
          }
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

// Dense per-token product on packed operands with TM x 192 tiles, two workgroups per CU:
// G * ceil(M/TM) * N/192 workgroups, N % 192 == 0; EPI_GELU or EPI_RESID.
template <int EPI, int TM>
__global__ __launch_bounds__(MFMA_THREADS, 2) void gemm_bf16_mfma_n192(GemmArgs p) {
  static_assert(EPI == EPI_GELU || EPI == EPI_RESID, "TM x 192 tiles serve the inference epilogues");
  static_assert(TM == 256 || TM == 128, "256- or 128-row tiles");
  using C = Pk3<TM>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[C::NS * C::SG];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + TM - 1) / TM, nNt = N / BN3;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  // bands of TILE_BAND row tiles, M-fastest inside a band (as in the 256 x 256 kernel)
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  // the tile's A blocks (packed row block, K/32 x 16 KB; a 128-row tile starts at the first or
  // second 8 KB half of each) and the token's whole W^T (pk_rows(N) rows; slices < 2^31
  // bytes, checked at launch)
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  const int nMb = (M + BM - 1) / BM;                    // packed 256-row blocks per token
  const int mb = mt / (BM / TM), half = mt % (BM / TM);  // block and half of this tile
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(static_cast<const uint16_t*>(p.A) + (size_t(g) * nMb + mb) * (size_t(blk) / 2) + size_t(half) * 4096,
                blk - uint32_t(half) * 8192u);
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
  f32x16_t acc[TM / 64][3];
  mfma_tile_pk3<TM>(acc, rA, rW, smem, lds0, K, nt, wave, lane);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue3<EPI, TM>(acc, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN3, mt * TM, wave, lane);
}

// ------------------------------------------ 256 x 384 tiles on eight waves, one per CU
// The 256 x 384 tile's single wave per SIMD leaves the matrix cores idle during its epilogue
// and during LDS reads that the ring does not hide; two 256 x 192 workgroups per CU fill
// those gaps but copy each A block twice.  Here one workgroup of eight waves takes a
// 256 x 384 tile as two groups of four: group 0 computes columns 0..191, group 1 columns
// 192..383, each wave a 128 x 96 part (4 x 3 blocks of 32 x 32, 192 AGPR accumulators), so
// a SIMD runs two waves and A is staged once for both halves.  A stage holds the 16 KB A
// block and the tile's 384 W^T rows (24 KB) as 40 pieces of 1 KB: wave w copies A pieces w
// and w + 8 and W^T pieces w, w + 8, w + 16 (rows 16 q .. 16 q + 15 of the tile), five
// copies per K step, in a 3-stage ring (120 KB).  The next step's copies are issued between
// the second sub-step's MFMAs (after products 1, 3, 5, 7 and 9 of its 12), where they keep
// the copy queue busy without stalling the LDS reads.  Measured at the 1B shape, B = 2048:
// GELU product 1.12 ms against 1.18 for 256 x 192 tiles two to a CU, residual product
// 0.98 ms against 1.05 for the four-wave 256 x 384 tile.  Per block the same MFMAs in the
// same K order as the other tile shapes, so the bits are the same.
constexpr int W8_THREADS = 512;
constexpr int W8_NS = 3;

// K loop of an eight-wave 256 x 384 tile.  GATHER_A: A is gathered from row-major rows as in
// mfma_tile_pk6; offA[c] is this lane's byte offset of piece wave + 8 c at K step 0.  NI < 4:
// only the wave's first NI row blocks hold rows; the others are neither read nor multiplied
// and their accumulators stay zero.  Copies and barriers are the same for every NI, so the
// waves of one workgroup may run different NI.
template <bool GATHER_A, int NI>
__device__ __forceinline__ void mfma_tile_w8(f32x16_t (&acc)[4][3], __amdgpu_buffer_rsrc_t rA,
                                             __amdgpu_buffer_rsrc_t rW, lds_u8* smem, uint32_t lds0, int K, int nt,
                                             int wave, int lane, const uint32_t (&offA)[2]) {
  static_assert(NI >= 0 && NI <= 4, "row blocks of a wave");
  constexpr int APW = 2;                     // A pieces per wave and K step
  constexpr int NCP = 5;                     // copies per wave and K step
  constexpr int SA = A_STAGE_BYTES;          // A part of a stage
  constexpr int SG = STAGE6_BYTES;           // stage bytes
  const int nk = K / BK;
  // W^T piece q = wave + 8 c holds rows 16 q .. 16 q + 15 of the tile (inside one 256-row
  // packed block, since 384 nt and 16 q are multiples of 16)
  uint32_t voffW[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int row = BN6 * nt + 16 * (wave + 8 * c);
    voffW[c] = uint32_t(row >> 8) * uint32_t(nk) * 16384u + uint32_t(row & 255) * 64u + uint32_t(lane) * 16u;
  }
  // copy c of K step kt into a stage; steps past the last re-read the last (never consumed)
  auto copy = [&](int kt, int stage, int c) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * SG;
    if (c < APW) {
      const uint32_t piece = uint32_t(wave + 8 * c);
      if constexpr (GATHER_A)
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), offA[c], rA, kt * BK * 2);
      else
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), piece * 1024u + uint32_t(lane) * 16u, rA,
                    kt * 16384);
    } else {
      const uint32_t q = uint32_t(wave + 8 * (c - APW));
      copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + SA + q * 1024u), voffW[c - APW], rW, kt * 16384);
    }
  };
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = kk * 2 + (lane >> 5);
    aoff[kk] = pk_lds_off(wm * 128 + (lane & 31), c);
    boff[kk] = uint32_t(SA) + pk_lds_off(grp * BN3 + wn * 96 + (lane & 31), c);
  }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  constexpr int NA = NI > 0 ? NI : 1;
  u32x4_t a0[NA], a1[NA], b[3];
  auto read_a = [&](u32x4_t (&a)[NA], const lds_u8* sp, int kk) {
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[kk] + i * 2048);
  };
  auto read_b = [&](const lds_u8* sp, int kk, int j) {
    if constexpr (NI > 0) b[j] = *reinterpret_cast<const lds_u32x4*>(sp + boff[kk] + j * 2048);
  };
  auto mm = [&](const u32x4_t (&a)[NA], int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                        __builtin_bit_cast(bf16x8_t, a[i]), acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
  for (int st = 0; st < W8_NS; ++st)
#pragma unroll
    for (int c = 0; c < NCP; ++c) copy(st, st, c);
  // step 0 has landed when at most the two later steps' copies (10) are outstanding
  asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  read_a(a0, smem, 0);
#pragma unroll
  for (int j = 0; j < 3; ++j) read_b(smem, 0, j);
  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * SG;
    const int nstage = stage + 1 == W8_NS ? 0 : stage + 1;
    // sub-step 0 (K columns 0..15 of the step) while the fragments of sub-step 1 are read
    read_a(a1, sp, 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
#pragma unroll
      for (int i = 0; i < NI; ++i) mm(a0, i, j);
      __builtin_amdgcn_sched_barrier(0);
      read_b(sp, 1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave has read this stage and step it + 1 has landed (the copies of step it + 2,
    // five per wave, may still be outstanding)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1 while step it + 3 is copied into the stage just consumed and the next
    // stage's sub-step 0 fragments are read; the copies go after products 1, 3, 5, 7, 9 of
    // the sub-step's twelve (by position, whether or not a row block is multiplied)
    const lds_u8* np = smem + nstage * SG;
    read_a(a0, np, 0);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < NI) mm(a1, i, j);
        const int q = 4 * j + i;
        if (q & 1 && q <= 9) {
          __builtin_amdgcn_sched_barrier(0);
          copy(it + W8_NS, stage, q / 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      read_b(np, 0, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Epilogue of an eight-wave 256 x 384 tile: each group of four waves stores its 256 x 192
// half as tile_epilogue3 does (32-column blocks staged through LDS, four lanes per row with
// eight columns each, 16 rows per pass), its staging rows after the other group's.  Tile row
// r is output row row_of(r) (-1: not stored); a wave's row blocks from nib on hold no rows
// and are skipped.  The arithmetic of each epilogue is that of tile_epilogue6.
template <int EPI, bool RM = false, typename RowOf>
__device__ __forceinline__ void tile_epilogue_w8(const f32x16_t (&acc)[4][3], float* smem_f, const GemmArgs& p,
                                                 int g, const bf16_t* bias_g, int n0, int wave, int lane,
                                                 RowOf row_of, int nib = 4) {
  const int M = p.M, N = p.N;
  const int wg = wave & 3;
  const int wrow0 = (wg >> 1) * 128, wcol0 = (wave >> 2) * BN3 + (wg & 1) * 96;
  float* st = smem_f + wave * 32 * LD3;
  const int col8 = (lane & 3) * 8;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int n = n0 + wcol0 + j * 32 + col8;
    float bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bias[e] = 0.f;
    if (bias_g) load8(bias_g + n, bias);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nib) break;  // row blocks past the rows (wave-uniform)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(st + (lane & 31) * LD3 + 8 * g4 + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
      // the staging rows are private to this wave, whose LDS operations complete in order
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int row = pass * 16 + (lane >> 2);
        const int m = row_of(wrow0 + i * 32 + row);
        float v[8];
        const float4 x0 = *reinterpret_cast<const float4*>(st + row * LD3 + col8);
        const float4 x1 = *reinterpret_cast<const float4*>(st + row * LD3 + col8 + 4);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        if (m >= 0) {
          const size_t rmo = size_t(g) * size_t(p.sc) + size_t(m) * size_t(p.ldc) + n;  // row-major
          if constexpr (EPI == EPI_GELU) {
            const size_t pko = size_t(g) * size_t(pk_rows(M)) * N + pk_off(m, n, N);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[e]);
            store8(static_cast<bf16_t*>(p.C) + pko, v);
          } else if constexpr (EPI == EPI_GELU_SAVE) {
            static_assert(RM, "the training epilogue writes row-major H and GELU'");
            float gd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf_and_grad(v[e] + bias[e], &gd[e]);
            store8(static_cast<bf16_t*>(p.U) + rmo, gd);
            store8(static_cast<bf16_t*>(p.C) + rmo, v);
          } else if constexpr (EPI == EPI_RESID) {
            const size_t pko = RM ? rmo : size_t(g) * size_t(pk_rows(M)) * N + pk_off(m, n, N);
            float rr[8];
            load8(static_cast<const bf16_t*>(p.R) + pko, rr);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] + bias[e] + rr[e];
            store8(static_cast<float*>(p.C) + rmo, v);
          } else if constexpr (EPI == EPI_MOE1) {
            // hidden rows in the packed layout, m a row of the group's tile-aligned blocks
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e] + bias[e]);
            store8(static_cast<bf16_t*>(p.C) + pk_off(m, n, N), v);
          } else {
            static_assert(EPI == EPI_MOE2, "an epilogue of the eight-wave tiles");
            const float gv = p.row_gate[m];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gv * (v[e] + bias[e]);
            store8(static_cast<bf16_t*>(p.C) + size_t(m) * size_t(N) + n, v);
          }
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

// Byte offsets of a lane's two gathered A pieces (wave and wave + 8) at K step 0: tile row
// r = pk_gather_row(piece, lane) is source row src(r) (negative: past the rows, read as zeros
// through an offset past the descriptor's end, `bytes`).
template <typename SrcRow>
__device__ __forceinline__ void w8_gather_offsets(uint32_t (&offA)[2], int wave, int lane, uint32_t row_bytes,
                                                  uint32_t bytes, SrcRow src) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = pk_gather_row(wave + 8 * c, lane);
    const uint32_t chunk16 = uint32_t(pk_gather_chunk(r, lane)) * 16u;
    const int s = src(r);
    offA[c] = s >= 0 ? uint32_t(s) * row_bytes + chunk16 : bytes;
  }
}

// Dense per-token product on packed operands with 256 x 384 tiles of eight waves:
// G * ceil(M/256) * N/384 workgroups of 512 threads, N % 384 == 0; EPI_GELU or EPI_RESID.
template <int EPI>
__global__ __launch_bounds__(W8_THREADS, 1) void gemm_bf16_mfma_w8(GemmArgs p) {
  static_assert(EPI == EPI_GELU || EPI == EPI_RESID, "eight-wave tiles serve the inference epilogues");
  static_assert(8 * 32 * LD3 * 4 <= W8_NS * STAGE6_BYTES, "epilogue staging fits in the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[W8_NS * STAGE6_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = N / BN6;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  // bands of TILE_BAND row tiles, M-fastest inside a band (as in the 256 x 256 kernel)
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  // the tile's A block (packed row block, K/32 x 16 KB) and the token's whole W^T
  // (pk_rows(N) rows; slices < 2^31 bytes, checked at launch)
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(static_cast<const uint16_t*>(p.A) + (size_t(g) * nMt + mt) * (size_t(blk) / 2), blk);
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
  f32x16_t acc[4][3];
  const uint32_t no_gather[2] = {0u, 0u};
  mfma_tile_w8<false, 4>(acc, rA, rW, smem, lds0, K, nt, wave, lane, no_gather);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  const int m0 = mt * BM;
  tile_epilogue_w8<EPI>(acc, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                        [&](int r) { return m0 + r < M ? m0 + r : -1; });
}

// Dense per-token product with row-major A (the training forward's saved S and H) and
// prepared W^T, 256 x 384 tiles: A rows are gathered straight into the packed LDS layout (the
// K loop of the Sparse-MoE kernel), the epilogue writes row-major outputs.  Per block the
// same MFMAs in the same K order as the row-major kernels, so the outputs are the same bits.
// G * ceil(M/256) * N/384 workgroups, N % 384 == 0, M * K * 2 < 2^31; EPI_GELU_SAVE or
// EPI_RESID.
template <int EPI>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_mfma_n384g(GemmArgs p) {
  static_assert(EPI == EPI_GELU_SAVE || EPI == EPI_RESID, "the training forward's epilogues");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[PK6_NS * STAGE6_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = N / BN6;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  // bands of TILE_BAND row tiles, M-fastest inside a band (as in the 256 x 256 kernel)
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  const int m0 = mt * BM;
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
  // A: the token's rows [M x K]; rows past M read as zeros (offset past the descriptor's end)
  const uint32_t row_bytes = uint32_t(K) * 2u, bytesA = uint32_t(M) * row_bytes;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(g) * size_t(p.sa), bytesA);
  uint32_t offA[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // piece wave + 4 c of the K step: tile row r, chunk pk_gather_chunk of its 64 bytes
    const int r = pk_gather_row(wave + 4 * c, lane);
    const uint32_t chunk16 = uint32_t(pk_gather_chunk(r, lane)) * 16u;
    offA[c] = m0 + r < M ? uint32_t(m0 + r) * row_bytes + chunk16 : bytesA;
  }
  f32x16_t accA[4][4], accV[4][2];
  mfma_tile_pk6<true, 4>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue6<EPI, 256, true>(accA, accV, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                                 [&](int r) { return m0 + r < M ? m0 + r : -1; });
}

// The training forward's products on eight-wave 256 x 384 tiles: gemm_bf16_mfma_n384g's
// operands and outputs, mfma_tile_w8's K loop with gathered A.  Same bits.
template <int EPI>
__global__ __launch_bounds__(W8_THREADS, 1) void gemm_bf16_mfma_w8g(GemmArgs p) {
  static_assert(EPI == EPI_GELU_SAVE || EPI == EPI_RESID, "the training forward's epilogues");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[W8_NS * STAGE6_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = N / BN6;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  const int m0 = mt * BM;
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
  // A: the token's rows [M x K]; rows past M read as zeros
  const uint32_t row_bytes = uint32_t(K) * 2u, bytesA = uint32_t(M) * row_bytes;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(g) * size_t(p.sa), bytesA);
  uint32_t offA[2];
  w8_gather_offsets(offA, wave, lane, row_bytes, bytesA, [&](int r) { return m0 + r < M ? m0 + r : -1; });
  f32x16_t acc[4][3];
  mfma_tile_w8<true, 4>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue_w8<EPI, true>(acc, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                              [&](int r) { return m0 + r < M ? m0 + r : -1; });
}

// Sparse-MoE grouped GEMM on prepared expert weights with 256 x 384 tiles: the persistent
// tile walk of gemm_bf16_moe (same device-built tile table, each XCD a contiguous range of
// tiles, row tiles fastest inside a group), the K loop of gemm_bf16_mfma_n384 and
// tile_epilogue6.  W is group g's W^T in the packed layout (pk_rows(N) x K, N % 384 == 0).
// Layer 1 gathers its A rows from S and writes the hidden rows in the packed layout, group g
// on the blocks tile_start[g] .. tile_start[g + 1] - 1 (its row tile mt on block
// tile_start[g] + mt); layer 2 reads those blocks as they are.  Same products in the same
// order as gemm_bf16_moe, so the two give the same bits.
template <int EPI>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_moe_n384(GemmArgs p) {
  static_assert(EPI == EPI_MOE1 || EPI == EPI_MOE2, "the Sparse-MoE epilogues");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[PK6_NS * STAGE6_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K, G = p.G;
  const int nNt = N / BN6;
  const int total = p.tile_start[G] * nNt;
  const int per_xcd = int(gridDim.x) / NUM_XCD;  // gridDim.x is a multiple of NUM_XCD
  const int xcd = int(blockIdx.x) % NUM_XCD, slot = int(blockIdx.x) / NUM_XCD;
  int lo, hi;
  moe_xcd_span(total, xcd, NUM_XCD, lo, hi);
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;

  for (int tile = lo + slot; tile < hi; tile += per_xcd) {
    int g, mt, nt;
    moe_tile_locate(p.tile_start, G, nNt, tile, g, mt, nt);
    const int row0 = p.group_start[g], rows = p.group_start[g + 1] - row0;
    const int m0 = mt * BM;
    // the tile's block of the packed hidden rows: groups start on whole 256-row blocks
    const int hblk = p.tile_start[g] + mt;
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
    // A: layer 1 gathers rows of S through the row list (rows past the group read as zeros:
    // offset past the descriptor's end); layer 2 reads the tile's packed block of hidden
    // rows, whose rows past the group are never stored
    uint32_t offA[4];
    __amdgpu_buffer_rsrc_t rA;
    if constexpr (EPI == EPI_MOE1) {
      const uint32_t row_bytes = uint32_t(K) * 2u;
      const uint32_t bytesA = uint32_t(p.a_rows) * row_bytes;
      rA = make_rsrc(p.A, bytesA);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // piece wave + 4 c of the K step: tile row r, chunk pk_gather_chunk of its 64 bytes
        const int r = pk_gather_row(wave + 4 * c, lane);
        const uint32_t chunk16 = uint32_t(pk_gather_chunk(r, lane)) * 16u;
        offA[c] = m0 + r < rows ? uint32_t(p.src_row[row0 + m0 + r]) * row_bytes + chunk16 : bytesA;
      }
    } else {
      rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(hblk) * (size_t(blk) / 2), blk);
#pragma unroll
      for (int c = 0; c < 4; ++c) offA[c] = 0u;
    }
    constexpr bool GA = EPI == EPI_MOE1;
    // row blocks of this wave (32 rows each) that hold rows of the group: 4 except in a
    // group's last row tile, where the MFMA work past the rows is skipped
    const int nib = __builtin_amdgcn_readfirstlane(max(0, min(4, (rows - m0 - (wave >> 1) * 128 + 31) / 32)));
    f32x16_t accA[4][4], accV[4][2];
    switch (nib) {
      case 4: mfma_tile_pk6<GA, 4>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 3: mfma_tile_pk6<GA, 3>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 2: mfma_tile_pk6<GA, 2>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 1: mfma_tile_pk6<GA, 1>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      default: mfma_tile_pk6<GA, 0>(accA, accV, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
    }
    const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
    // output rows: layer 1 the packed hidden block, layer 2 the compacted expert rows
    tile_epilogue6<EPI>(accA, accV, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                        [&](int r) { return m0 + r < rows ? (GA ? hblk * BM + r : row0 + m0 + r) : -1; }, nib);
    // every wave is done with its staging rows before the next tile's copies reuse the ring
    __syncthreads();
  }
}

// The Sparse-MoE grouped products on eight-wave 256 x 384 tiles: gemm_bf16_moe_n384's tile
// walk, operands and outputs, mfma_tile_w8's K loop.  A wave's row blocks past the group's
// rows are skipped as there.  Same bits.
template <int EPI>
__global__ __launch_bounds__(W8_THREADS, 1) void gemm_bf16_moe_w8(GemmArgs p) {
  static_assert(EPI == EPI_MOE1 || EPI == EPI_MOE2, "the Sparse-MoE epilogues");
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[W8_NS * STAGE6_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, K = p.K, G = p.G;
  const int nNt = N / BN6;
  const int total = p.tile_start[G] * nNt;
  const int per_xcd = int(gridDim.x) / NUM_XCD;  // gridDim.x is a multiple of NUM_XCD
  const int xcd = int(blockIdx.x) % NUM_XCD, slot = int(blockIdx.x) / NUM_XCD;
  int lo, hi;
  moe_xcd_span(total, xcd, NUM_XCD, lo, hi);
  const uint32_t blk = uint32_t(K / BK) * 16384u;
  const uint32_t wbytes = uint32_t(pk_rows(N) / 256) * blk;
  constexpr bool GA = EPI == EPI_MOE1;

  for (int tile = lo + slot; tile < hi; tile += per_xcd) {
    int g, mt, nt;
    moe_tile_locate(p.tile_start, G, nNt, tile, g, mt, nt);
    const int row0 = p.group_start[g], rows = p.group_start[g + 1] - row0;
    const int m0 = mt * BM;
    const int hblk = p.tile_start[g] + mt;  // the tile's block of the packed hidden rows
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * (size_t(wbytes) / 2), wbytes);
    uint32_t offA[2] = {0u, 0u};
    __amdgpu_buffer_rsrc_t rA;
    if constexpr (GA) {
      const uint32_t row_bytes = uint32_t(K) * 2u;
      const uint32_t bytesA = uint32_t(p.a_rows) * row_bytes;
      rA = make_rsrc(p.A, bytesA);
      w8_gather_offsets(offA, wave, lane, row_bytes, bytesA,
                        [&](int r) { return m0 + r < rows ? p.src_row[row0 + m0 + r] : -1; });
    } else {
      rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(hblk) * (size_t(blk) / 2), blk);
    }
    const int nib =
        __builtin_amdgcn_readfirstlane(max(0, min(4, (rows - m0 - ((wave >> 1) & 1) * 128 + 31) / 32)));
    f32x16_t acc[4][3];
    switch (nib) {
      case 4: mfma_tile_w8<GA, 4>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 3: mfma_tile_w8<GA, 3>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 2: mfma_tile_w8<GA, 2>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      case 1: mfma_tile_w8<GA, 1>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
      default: mfma_tile_w8<GA, 0>(acc, rA, rW, smem, lds0, K, nt, wave, lane, offA); break;
    }
    const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
    tile_epilogue_w8<EPI>(acc, reinterpret_cast<float*>(smem_g), p, g, bias_g, nt * BN6, wave, lane,
                          [&](int r) { return m0 + r < rows ? (GA ? hblk * BM + r : row0 + m0 + r) : -1; }, nib);
    // every wave is done with its staging rows before the next tile's copies reuse the ring
    __syncthreads();
  }
}

// ------------------------------------------------------------- MXFP8 products
// The prepared-operand K loop with 8-bit operands: a K step is 64 values, so a stage holds
// the same 16 KB per operand (256 rows x 64 E4M3 codes, one contiguous block of the MXFP8
// layout) plus the step's scales (512 bytes per operand, one 32-bit LDS read per lane and
// operand).  Each 32 x 32 block takes one v_mfma_scale_f32_32x32x64_f8f6f4 per step: lane l
// supplies row l % 32 of each operand, h = l / 32: bytes 0-15 are k 16 h .. 16 h + 15 (of
// the step's first 32-value scale block), bytes 16-31 are k 32 + 16 h .. 32 + 16 h + 15 (of
// the second), i.e. chunks h and h + 2 of the row (two 16-byte LDS reads); the scale that
// lanes of half h supply (the byte the instruction selects) is that of scale block h.  The
// W fragment goes first, as in the bf16 loop, so the accumulator layout (and the epilogue)
// is the same.  Per stage and wave: 8 code copies of 1 KB and one scale copy of 256 bytes
// (waves 0, 1: the two halves of A's scales; waves 2, 3: W's).
constexpr int MX_BK = 64;
constexpr int MX_CODE_BYTES = 16384;                         // one operand's codes per stage
constexpr int MX_STAGE_BYTES = 2 * MX_CODE_BYTES + 1024;     // + both operands' scales
constexpr int MX_COPIES = 9;                                 // LDS-destination loads per wave per step

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// One LDS-destination buffer load of 4 bytes per lane: 64 lanes x 4 B to lds_dst + 4 * lane.
__device__ __forceinline__ void copy_to_lds_b32(uint32_t lds_dst, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc,
                                                int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_dst), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

struct MxFrags {
  u32x4_t a[4][2];  // A rows of the 4 row blocks: 32 codes each (two chunks)
  u32x4_t b[4][2];  // W^T rows (output columns) of the 4 column blocks
  uint32_t sa, sw;  // scale bytes of the 4 row blocks / 4 column blocks
};

template <int I, int J>
__device__ __forceinline__ void mx_mma(f32x16_t (&acc)[4][4], const MxFrags& f) {
  const u32x4_t a0 = f.a[I][0], a1 = f.a[I][1], b0 = f.b[J][0], b1 = f.b[J][1];
  const i32x8_t a = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
  const i32x8_t b = {int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
  // format 0 = FP8 E4M3 for both operands; scale byte J of sw for the first, I of sa for the second
  acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[I][J], 0, 0, J, int(f.sw), I, int(f.sa));
}

// the 16 products of a step, in 2 halves of 8 (blocks (i, j) with q = 4 i + j)
template <int H>
__device__ __forceinline__ void mx_half(f32x16_t (&acc)[4][4], const MxFrags& f) {
  mx_mma<2 * H, 0>(acc, f);
  mx_mma<2 * H, 1>(acc, f);
  mx_mma<2 * H, 2>(acc, f);
  mx_mma<2 * H, 3>(acc, f);
  mx_mma<2 * H + 1, 0>(acc, f);
  mx_mma<2 * H + 1, 1>(acc, f);
  mx_mma<2 * H + 1, 2>(acc, f);
  mx_mma<2 * H + 1, 3>(acc, f);
}

__device__ __forceinline__ void mfma_tile_mx(f32x16_t (&acc)[4][4], __amdgpu_buffer_rsrc_t rA,
                                             __amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rS, lds_u8* smem,
                                             uint32_t lds0, int K, int wave, int lane) {
  const int nk = K / MX_BK;
  // copy q (0..8) of K step kt into ring stage `stage`; steps past the end reload the last
  auto copy = [&](int kt, int stage, int q) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * MX_STAGE_BYTES;
    if (q < 8) {
      const uint32_t piece = uint32_t(4 * wave + (q & 3));
      const uint32_t voff = piece * 1024u + uint32_t(lane) * 16u;
      if (q < 4) copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + piece * 1024u), voff, rA, kt * MX_CODE_BYTES);
      else copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + MX_CODE_BYTES + piece * 1024u), voff, rW,
                       kt * MX_CODE_BYTES);
    } else {
      const uint32_t voff = uint32_t(wave & 1) * 256u + uint32_t(lane) * 4u;
      copy_to_lds_b32(__builtin_amdgcn_readfirstlane(sbase + 2 * MX_CODE_BYTES + uint32_t(wave) * 256u), voff, rS,
                      kt * 512);
    }
  };
  const int wm = wave >> 1, wn = wave & 1, hk = lane >> 5;
  uint32_t aoff[4][2], boff[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = wm * 128 + i * 32 + (lane & 31);
      aoff[i][c] = pk_lds_off(m, hk + 2 * c);
      const int n = wn * 128 + i * 32 + (lane & 31);
      boff[i][c] = uint32_t(MX_CODE_BYTES) + pk_lds_off(n, hk + 2 * c);
    }
  const uint32_t sa_off = uint32_t(2 * MX_CODE_BYTES + wm * 256 + lane * 4);
  const uint32_t sw_off = uint32_t(2 * MX_CODE_BYTES + 512 + wn * 256 + lane * 4);
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  auto read_frags = [&](MxFrags& f, const lds_u8* sp) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f.a[i][c] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[i][c]);
        f.b[i][c] = *reinterpret_cast<const lds_u32x4*>(sp + boff[i][c]);
      }
    f.sa = *reinterpret_cast<const lds_u32*>(sp + sa_off);
    f.sw = *reinterpret_cast<const lds_u32*>(sp + sw_off);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // prologue: steps 0..PK_NS-1; wait for step 0 (MX_COPIES loads per step)
#pragma unroll
  for (int st = 0; st < PK_NS; ++st)
#pragma unroll
    for (int q = 0; q < MX_COPIES; ++q) copy(st, st, q);
  asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
  MxFrags f0, f1;
  read_frags(f0, smem);
  // One step: `cur` holds step it (read during the previous step).  After the barrier step
  // it+1 is visible (the MX_COPIES loads of step it+2 may be outstanding) and every wave is
  // done reading stage(it), which then takes step it+PK_NS.
  auto step = [&](MxFrags& cur, MxFrags& nxt, int it, int stage) {
    const int nstage = stage + 1 == PK_NS ? 0 : stage + 1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_frags(nxt, smem + nstage * MX_STAGE_BYTES);
    mx_half<0>(acc, cur);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<2, 0>(acc, cur);
    copy(it + PK_NS, stage, 0);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<2, 1>(acc, cur);
    copy(it + PK_NS, stage, 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<2, 2>(acc, cur);
    copy(it + PK_NS, stage, 2);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<2, 3>(acc, cur);
    copy(it + PK_NS, stage, 3);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<3, 0>(acc, cur);
    copy(it + PK_NS, stage, 4);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<3, 1>(acc, cur);
    copy(it + PK_NS, stage, 5);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<3, 2>(acc, cur);
    copy(it + PK_NS, stage, 6);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<3, 3>(acc, cur);
    copy(it + PK_NS, stage, 7);
    copy(it + PK_NS, stage, 8);
    __builtin_amdgcn_sched_barrier(0);
    return nstage;
  };
  int stage = 0;
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    stage = step(f0, f1, it, stage);
    stage = step(f1, f0, it + 1, stage);
  }
  if (it < nk) step(f0, f1, it, stage);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

template <int EPI>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_mx_mfma(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[PK_NS * MX_STAGE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + BM - 1) / BM, nNt = (N + BN - 1) / BN;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  int mt, nt;
  band_tile(rem, nMt, nNt, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const uint32_t nk = uint32_t(K / MX_BK);
  const uint8_t* A = static_cast<const uint8_t*>(p.A) + (size_t(g) * nMt + mt) * (size_t(nk) * MX_CODE_BYTES);
  const uint8_t* W = static_cast<const uint8_t*>(p.W) + (size_t(g) * nNt + nt) * (size_t(nk) * MX_CODE_BYTES);
  const uint8_t* SA = static_cast<const uint8_t*>(p.A_scale) + (size_t(g) * nMt + mt) * (size_t(nk) * 512);
  const uint8_t* SW = static_cast<const uint8_t*>(p.W_scale) + (size_t(g) * nNt + nt) * (size_t(nk) * 512);
  f32x16_t acc[4][4];
  mfma_tile_mx(acc, make_rsrc(A, nk * MX_CODE_BYTES), make_rsrc(W, nk * MX_CODE_BYTES),
               make_rsrc(wave < 2 ? SA : SW, nk * 512u), smem, lds0, K, wave, lane);
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue<EPI, 4, 4, true>(acc, reinterpret_cast<float*>(smem_g), p, bias_g, n0, (wave >> 1) * 128,
                                 (wave & 1) * 128, wave, lane, g, [&](int m) { return m0 + m < M ? m0 + m : -1; });
}

// Sparse-MoE grouped GEMM.  Group g has rows group_start[g] .. group_start[g+1]-1 of the
// compacted row space and tile_start[g+1] - tile_start[g] row tiles; the grid is a fixed set
// of workgroups that walk the tile space (its size is only known on the device).  Each XCD
// takes a contiguous range of tiles; within a group tiles run M-fastest, so a group's
// expert weights are reused across its row tiles.
template <int EPI>
__global__ __launch_bounds__(MFMA_THREADS, 1) void gemm_bf16_moe(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[NS * STAGE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, G = p.G;
  const int nNt = (N + BN - 1) / BN;
  const int total = p.tile_start[G] * nNt;
  const int per_xcd = int(gridDim.x) / NUM_XCD;  // gridDim.x is a multiple of NUM_XCD
  const int xcd = int(blockIdx.x) % NUM_XCD, slot = int(blockIdx.x) / NUM_XCD;
  int lo, hi;
  moe_xcd_span(total, xcd, NUM_XCD, lo, hi);
  const uint32_t bytesW = uint32_t(K) * uint32_t(N) * 2u;

  for (int tile = lo + slot; tile < hi; tile += per_xcd) {
    int g, mt, nt;
    moe_tile_locate(p.tile_start, G, nNt, tile, g, mt, nt);
    const int row0 = p.group_start[g], rows = p.group_start[g + 1] - row0;
    const int m0 = mt * BM, n0 = nt * BN;

    TileSrc ts;
    ts.rW = make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * K * N, bytesW);
    if constexpr (EPI == EPI_MOE1) {
      // rows gathered from A = S [a_rows, K] through src_row
      const uint32_t bytesA = uint32_t(p.a_rows) * uint32_t(K) * 2u;
      ts.rA = make_rsrc(p.A, bytesA);
      tile_offsets(ts, wave, lane, n0, N,
                   [&](int r, int cbytes) {
                     return (m0 + r < rows) ? uint32_t(p.src_row[row0 + m0 + r]) * uint32_t(K) * 2u + uint32_t(cbytes)
                                            : bytesA;
                   },
                   bytesW);
    } else {
      // rows of A are this group's compacted rows, contiguous
      const uint32_t bytesA = uint32_t(rows) * uint32_t(K) * 2u;
      ts.rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(row0) * K, bytesA);
      tile_offsets(ts, wave, lane, n0, N,
                   [&](int r, int cbytes) {
                     return (m0 + r < rows) ? uint32_t(m0 + r) * uint32_t(K) * 2u + uint32_t(cbytes) : bytesA;
                   },
                   bytesW);
    }
    f32x16_t acc[4][4];
    mfma_tile(acc, ts, smem, lds0, K, N, wave, lane);
    const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
    tile_epilogue<EPI, 4, 4, false>(acc, reinterpret_cast<float*>(smem_g), p, bias_g, n0, (wave >> 1) * 128,
                                    (wave & 1) * 128, wave, lane, 0,
                                    [&](int m) { return m0 + m < rows ? row0 + m0 + m : -1; });
  }
}

// ----------------------------------------------------------- small-batch kernel
// Tiles of 64 rows x 256 columns for few rows per token (serving batches): the weight
// panel dominates the bytes, and a 256-row tile would spend three quarters of its MFMA
// work on rows that do not exist.  4 waves side by side, each 64 x 64 (2 x 2 blocks);
// K steps of 32 through a 4-stage ring of 20 KB (A 64 x 32, W 32 x 256), so two workgroups
// share a CU and their copy streams overlap.  Same copy, swizzle and wait scheme as the
// 256 x 256 kernel: 5 loads per wave per K step (1 of A, 4 of W).
// SBN = 128 (packed operands only): 64 x 128 tiles, waves of 64 x 32, 3 loads per wave per
// K step (the tile's W^T rows are one 8 KB half of each packed 256-row block), for launches
// whose 64 x 256 tiles would load the CUs unevenly (see narrow_small_tiles).
constexpr int SM_BM = 64;
constexpr int SM_A_BYTES = SM_BM * BK * 2;                 // 4 KB, rows of 64 B

template <int EPI, bool PK, int SBN = 256>
__global__ __launch_bounds__(MFMA_THREADS, 2) void gemm_bf16_mfma_m64(GemmArgs p) {
  static_assert(SBN == 256 || (SBN == 128 && PK), "64 x 128 tiles need packed operands");
  constexpr int SM_STAGE_BYTES = SM_A_BYTES + BK * SBN * 2;  // + 16 KB or 8 KB of W
  constexpr int WPW = SBN / 64;                               // W pieces per wave and K step
  constexpr int SM_COPIES = 1 + WPW;
  constexpr int NJ = SBN / 128;                               // column blocks per wave
  __shared__ __attribute__((aligned(1024))) unsigned char smem_g[NS * SM_STAGE_BYTES];
  lds_u8* const smem = (lds_u8*)smem_g;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int nMt = (M + SM_BM - 1) / SM_BM, nNt = (N + SBN - 1) / SBN;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int g = id / (nMt * nNt);
  const int rem = id - g * nMt * nNt;
  const int nt = rem / nMt, mt = rem - nt * nMt;
  const int m0 = mt * SM_BM, n0 = nt * SBN;
  const int nk = K / BK;

  __amdgpu_buffer_rsrc_t rA, rW;
  // row-major operands: copy 0 takes A rows 16 w .. 16 w + 15 (lane q takes chunk q % 4 of
  // row q / 4, swizzled), copies 1..4 W k rows 8 w + 2 (c - 1) and +1, as in the 256 x 256
  // kernel.  Packed operands: copy 0 is piece w of the 4 KB of the tile's 64 A rows in the
  // step's 16 KB block, copies 1..4 pieces 4 w .. 4 w + 3 of the 16 KB W^T block.
  uint32_t offA, offW[4];
  if constexpr (PK) {
    const uint32_t blk = uint32_t(nk) * 16384u;
    const int64_t row_blocks = pk_rows(M) / 256;
    const int nNb = int(pk_rows(N) / 256);                         // packed W^T blocks
    const int wb = nt / (256 / SBN), wh = nt % (256 / SBN);          // block, half of it
    rA = make_rsrc(static_cast<const uint16_t*>(p.A) + (size_t(g) * row_blocks + m0 / 256) * (size_t(blk) / 2), blk);
    rW = make_rsrc(static_cast<const uint16_t*>(p.W) + (size_t(g) * nNb + wb) * (size_t(blk) / 2) + size_t(wh) * 4096,
                   blk - uint32_t(wh) * 8192u);
    offA = uint32_t(m0 % 256) * 64u + uint32_t(wave) * 1024u + uint32_t(lane) * 16u;
#pragma unroll
    for (int a = 0; a < 4; ++a) offW[a] = uint32_t(WPW * wave + (a < WPW ? a : 0)) * 1024u + uint32_t(lane) * 16u;
  } else {
    const uint32_t lda = uint32_t(p.lda);
    const uint32_t bytesA = (uint32_t(M - 1) * lda + uint32_t(K)) * 2u, bytesW = uint32_t(K) * uint32_t(N) * 2u;
    rA = make_rsrc(static_cast<const uint16_t*>(p.A) + size_t(g) * size_t(p.sa), bytesA);
    rW = make_rsrc(static_cast<const uint16_t*>(p.W) + size_t(g) * K * N, bytesW);
    const int r = 16 * wave + (lane >> 2);
    const int c = (lane & 3) ^ swz_a(r);
    offA = (m0 + r < M) ? uint32_t(m0 + r) * lda * 2u + uint32_t(c * 16) : bytesA;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int kr = 8 * wave + 2 * a + (lane >> 5);
      const int col = n0 + (((lane & 31) ^ swz_w(kr)) * 8);
      offW[a] = col < N ? (uint32_t(kr) * uint32_t(N) + uint32_t(col)) * 2u : bytesW;
    }
  }
  auto copy = [&](int kt, int stage, int q) {
    kt = kt < nk ? kt : nk - 1;
    const uint32_t sbase = lds0 + uint32_t(stage) * SM_STAGE_BYTES;
    if constexpr (PK) {
      if (q == 0) {
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + uint32_t(wave) * 1024u), offA, rA, kt * 16384);
      } else {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + SM_A_BYTES + uint32_t(WPW * wave + q - 1) * 1024u);
        copy_to_lds(dst, offW[q - 1], rW, kt * 16384);
      }
    } else {
      if (q == 0) {
        copy_to_lds(__builtin_amdgcn_readfirstlane(sbase + uint32_t(16 * wave) * 64u), offA, rA, kt * BK * 2);
      } else {
        const uint32_t dst =
            __builtin_amdgcn_readfirstlane(sbase + SM_A_BYTES + uint32_t(8 * wave + 2 * (q - 1)) * 512u);
        copy_to_lds(dst, offW[q - 1], rW, kt * BK * N * 2);
      }
    }
  };

  uint32_t aoff[2][2], boff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = i * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      aoff[kk][i] = uint32_t(m * 64 + ((c ^ swz_a(m)) << 4));
      if constexpr (PK) {
        const int n = wave * (SBN / 4) + i * 32 + (lane & 31);
        boff[kk][i] = uint32_t(SM_A_BYTES) + pk_lds_off(n, c);
      } else {
        const int kb = 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int n = wave * 64 + i * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        boff[kk][i] = uint32_t(SM_A_BYTES + kb * 512 + (((n >> 3) ^ swz_w(kb)) << 4) + (n & 7) * 2);
      }
    }
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  struct SmFrags {
    u32x4_t a[2];
    u32x4_t b[NJ];  // W columns of the NJ column blocks: 8 bf16 each
  };
  auto read_frags = [&](SmFrags& f, const lds_u8* sp, int kk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = *reinterpret_cast<const lds_u32x4*>(sp + aoff[kk][i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (PK) {
        f.b[j] = *reinterpret_cast<const lds_u32x4*>(sp + boff[kk][j]);
      } else {
        const lds_u8* q = sp + boff[0][j] + kk * 16 * 512;
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q));
        const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * 512)));
        f.b[j] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      }
    }
  };
  f32x16_t acc[2][NJ];
  auto mfma4 = [&](const SmFrags& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.b[j]),
                                                            __builtin_bit_cast(bf16x8_t, f.a[i]), acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Prologue: K steps 0..NS-1; wait for step 0 (SM_COPIES loads per step).
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int q = 0; q < SM_COPIES; ++q) copy(st, st, q);
  static_assert(NS == 4, "the wait counts below assume a 4-stage ring");
  if constexpr (SM_COPIES == 5)
    asm volatile("s_waitcnt vmcnt(15)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
  SmFrags f0, f1;
  read_frags(f0, smem, 0);
  int stage = 0;
  for (int it = 0; it < nk; ++it) {
    const lds_u8* sp = smem + stage * SM_STAGE_BYTES;
    const int nstage = stage + 1 == NS ? 0 : stage + 1;
    read_frags(f1, sp, 1);
    mfma4(f0);
    // step it+1 visible (the loads of the two steps after it may be outstanding); this
    // stage free for step it+NS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SM_COPIES == 5)
      asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_frags(f0, smem + nstage * SM_STAGE_BYTES, 0);
    mfma4(f1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < SM_COPIES; ++q) copy(it + NS, stage, q);
    __builtin_amdgcn_sched_barrier(0);
    stage = nstage;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const bf16_t* bias_g = p.bias ? static_cast<const bf16_t*>(p.bias) + size_t(g) * N : nullptr;
  tile_epilogue<EPI, 2, NJ, PK>(acc, reinterpret_cast<float*>(smem_g), p, bias_g, n0, 0, wave * (SBN / 4), wave,
                                lane, g, [&](int m) { return m0 + m < M ? m0 + m : -1; });
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
  const T* A = static_cast<const T*>(p.A) + size_t(g) * size_t(p.sa);
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
      const size_t a_at = p.at ? size_t(kk) * size_t(p.lda) + row : size_t(row) * size_t(p.lda) + kk;
      As[ak][am] = (row < M && kk < K) ? load1(A + a_at) : 0.f;
      const int bk = e / GT, bn = e % GT;
      const int kr = k0 + bk, col = n0 + bn;
      const size_t w_at = p.bt ? size_t(col) * K + kr : size_t(kr) * N + col;
      Bs[bk][bn] = (kr < K && col < N) ? load1(W + w_at) : 0.f;
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
      const size_t off = size_t(g) * size_t(p.sc) + size_t(m) * size_t(p.ldc) + n;
      if constexpr (EPI == EPI_GELU) {
        store1(static_cast<T*>(p.C) + off, gelu_erf(acc[i][j] + bias));
      } else if constexpr (EPI == EPI_GELU_SAVE) {
        float gd;
        store1(static_cast<T*>(p.C) + off, gelu_erf_and_grad(acc[i][j] + bias, &gd));
        store1(static_cast<T*>(p.U) + off, gd);
      } else if constexpr (EPI == EPI_GELU_BWD) {
        store1(static_cast<T*>(p.C) + off, acc[i][j] * load1(static_cast<const T*>(p.R) + off));
      } else if constexpr (EPI == EPI_RESID32) {
        static_cast<float*>(p.C)[off] = acc[i][j] + static_cast<const float*>(p.R)[off];
      } else if constexpr (EPI == EPI_STORE32) {
        static_cast<float*>(p.C)[off] = acc[i][j];
      } else if constexpr (EPI == EPI_BIAS) {
        store1(static_cast<T*>(p.C) + off, acc[i][j] + bias);
      } else {
        static_cast<float*>(p.C)[off] = acc[i][j] + bias + load1(static_cast<const T*>(p.R) + off);
      }
    }
  }
}

}  // namespace

bool gemm_uses_mfma(int dtype, int M, int N, int K, int64_t lda, int at, int bt) {
  const uint64_t lim = uint64_t(1) << 31;
  if (dtype != DT_BF16 || N % 8 != 0 || uint64_t(K) * N * 2 >= lim) return false;
  if (at) {
    // k rows of A are whole 16-byte chunks; the K tail loads zeros; with bt as well the
    // row-tile W needs K % 32 (no kernel takes both)
    const uint64_t ld = lda > 0 ? uint64_t(lda) : uint64_t(M);
    return !bt && M % 8 == 0 && ld % 8 == 0 && ld >= uint64_t(M) && uint64_t(K) * ld * 2 < lim;
  }
  const uint64_t ld = lda > 0 ? uint64_t(lda) : uint64_t(K);
  const uint64_t spanA = M > 0 ? (uint64_t(M - 1) * ld + uint64_t(K)) * 2 : 0;
  return K % BK == 0 && ld % 8 == 0 && spanA < lim;
}

hipError_t gemm_init() { return hipSuccess; }

bool gemm_packed_w_supported(int64_t M, int64_t N, int64_t K) {
  const uint64_t lim = uint64_t(1) << 31;
  return M > 0 && N > 0 && K > 0 && N % BN6 == 0 && K % BK == 0 && uint64_t(M) * uint64_t(K) * 2u < lim &&
         uint64_t(pk_rows(N)) * uint64_t(K) * 2u < lim;
}

bool gemm_moe_supported(int N, int K, int64_t a_rows, bool packed) {
  const uint64_t lim = uint64_t(1) << 31;
  if (packed && (N % BN6 != 0 || uint64_t(pk_rows(N)) * K * 2 >= lim)) return false;
  return K % BK == 0 && N % 8 == 0 && uint64_t(a_rows) * K * 2 < lim && uint64_t(K) * N * 2 < lim &&
         uint64_t(a_rows) * N * 2 < lim;
}

// The training forward's and the Sparse-MoE products on prepared weights run eight-wave
// 256 x 384 tiles; RMX_WIDE_TILES=always keeps them on the four-wave ones (tests and tuning;
// read at each launch; the same bits).
static bool four_wave_tiles() {
  const char* force = getenv("RMX_WIDE_TILES");
  return force && strcmp(force, "always") == 0;
}

hipError_t launch_gemm_moe(int epi, const GemmArgs& args, hipStream_t stream) {
  if (args.G == 0) return hipSuccess;
  GemmArgs a = args;  // outputs are the compacted rows [rows, N]
  a.ldc = a.N;
  a.sc = 0;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int grid = ((cus + NUM_XCD - 1) / NUM_XCD) * NUM_XCD;  // one workgroup per CU, whole XCDs
  if (a.packed) {
    if (a.N % BN6 != 0) return hipErrorInvalidValue;
    if (four_wave_tiles()) {
      if (epi == EPI_MOE1)
        hipLaunchKernelGGL((gemm_bf16_moe_n384<EPI_MOE1>), dim3(grid), dim3(MFMA_THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_bf16_moe_n384<EPI_MOE2>), dim3(grid), dim3(MFMA_THREADS), 0, stream, a);
    } else if (epi == EPI_MOE1) {
      hipLaunchKernelGGL((gemm_bf16_moe_w8<EPI_MOE1>), dim3(grid), dim3(W8_THREADS), 0, stream, a);
    } else {
      hipLaunchKernelGGL((gemm_bf16_moe_w8<EPI_MOE2>), dim3(grid), dim3(W8_THREADS), 0, stream, a);
    }
  } else if (epi == EPI_MOE1) {
    hipLaunchKernelGGL((gemm_bf16_moe<EPI_MOE1>), dim3(grid), dim3(MFMA_THREADS), 0, stream, a);
  } else {
    hipLaunchKernelGGL((gemm_bf16_moe<EPI_MOE2>), dim3(grid), dim3(MFMA_THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

namespace {

// Tile shape of a packed-operand product with the GELU or residual epilogue.  Each shape's
// cost is its number of rounds times the measured duration of one round of its tiles on the
// whole chip, relative to the others (1B shapes, K = 1536 and 6144; durations in units of
// about 2.8 us at K = 1536):
//   256 x 256: 20 per round of CUs tiles          256 x 384: 28 per round of CUs tiles
//   128 x 384: 17 per round of CUs tiles          (N % 384 == 0 for both)
//   256 x 192, two per CU: 27 per round of 2 CUs tiles (the GELU product only: for the
//       residual product at B = 2048 it is level with 256 x 384, 1.04 against 1.03 ms)
//   128 x 192, two per CU: 17 per round of 2 CUs tiles, 12 when the launch holds at most
//       one tile per CU (RankMixer-100M GEMM2, B = 512: 256 tiles, 56 us against 77 us for
//       its 128 x 384 tiles, which leave half of the CUs idle)
//   256 x 384 on eight waves: 26 per round of CUs tiles (1B, B = 2048: GELU product 1.12
//       against 1.18 ms on 256 x 192 tiles, residual product 0.98 against 1.05 ms)
// The fewest units win; ties go to the shape listed first.  384-wide tiles need
// N % 384 == 0, 192-wide ones N % 192 == 0, all of them a token's packed W^T below 2^31
// bytes (their buffer descriptor spans it).
// The environment variable RMX_WIDE_TILES = always / half / pair / pairhalf / wide8 / never
// forces 256 x 384, 128 x 384, 256 x 192, 128 x 192, 256 x 384 on eight waves or 256 x 256
// (tests and tuning; read at each launch; a shape N does not divide falls back to
// 256 x 256); all give the same bits.
enum TileShape {
  TILES_256 = 0,
  TILES_256x384 = 1,
  TILES_128x384 = 2,
  TILES_256x192 = 3,
  TILES_128x192 = 4,
  TILES_256x384w8 = 5
};

TileShape pick_tiles(const GemmArgs& a, int epi) {
  const char* force = getenv("RMX_WIDE_TILES");
  const bool w_ok = uint64_t(pk_rows(a.N)) * uint64_t(a.K) * 2u < (uint64_t(1) << 31);
  const bool n384 = w_ok && a.N % BN6 == 0, n192 = w_ok && a.N % BN3 == 0;
  if (force) {
    if (strcmp(force, "never") == 0) return TILES_256;
    if (strcmp(force, "always") == 0) return n384 ? TILES_256x384 : TILES_256;
    if (strcmp(force, "half") == 0) return n384 ? TILES_128x384 : TILES_256;
    if (strcmp(force, "pair") == 0) return n192 ? TILES_256x192 : TILES_256;
    if (strcmp(force, "pairhalf") == 0) return n192 ? TILES_128x192 : TILES_256;
    if (strcmp(force, "wide8") == 0) return n384 ? TILES_256x384w8 : TILES_256;
  }
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t G = a.G, m256 = (a.M + BM - 1) / BM, m128 = (a.M + 127) / 128;
  auto rounds = [&](int64_t tiles, int64_t slots) { return (tiles + slots - 1) / slots; };
  TileShape best = TILES_256;
  int64_t best_cost = 20 * rounds(G * m256 * ((a.N + BN - 1) / BN), cus);
  auto consider = [&](TileShape s, int64_t cost) {
    if (cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  };
  if (n384) {
    consider(TILES_256x384, 28 * rounds(G * m256 * (a.N / BN6), cus));
    consider(TILES_256x384w8, 26 * rounds(G * m256 * (a.N / BN6), cus));
    consider(TILES_128x384, 17 * rounds(G * m128 * (a.N / BN6), cus));
  }
  if (n192) {
    if (epi == EPI_GELU) consider(TILES_256x192, 27 * rounds(G * m256 * (a.N / BN3), 2 * int64_t(cus)));
    const int64_t t = G * m128 * (a.N / BN3);
    consider(TILES_128x192, t <= cus ? 12 : 17 * rounds(t, 2 * int64_t(cus)));
  }
  return best;
}

// 64-row tiles 128 columns wide (packed products) where the 256-wide ones number between
// one and two per CU, so that some CUs would run two and others one: the narrow tiles then
// spread evenly (measured at the 1B shapes, B = 128, GEMM2: 384 wide tiles 184 us, 768
// narrow ones 169 us).  With fewer wide tiles than CUs the narrow ones are slower (B = 64,
// GEMM2: 126 against 137 us): a workgroup streams its weight panel at a rate set by the
// bytes its ring keeps in flight, which the narrow tile halves.  RMX_NARROW_TILES = always /
// never forces the choice (tests and tuning; read at each launch); both give the same bits.
bool narrow_small_tiles(const GemmArgs& a) {
  const char* force = getenv("RMX_NARROW_TILES");
  if (force && strcmp(force, "never") == 0) return false;
  if (force && strcmp(force, "always") == 0) return true;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t tiles = int64_t(a.G) * ((a.M + SM_BM - 1) / SM_BM) * ((a.N + BN - 1) / BN);
  return tiles >= int64_t(cus) && tiles < 2 * int64_t(cus);
}

template <bool PK>
hipError_t launch_dense_mfma(int epi, const GemmArgs& a, hipStream_t stream) {
  if (a.M <= GEMM_SMALL_M) {
    if (PK && (epi == EPI_GELU || epi == EPI_RESID) && narrow_small_tiles(a)) {
      const int tiles = a.G * ((a.M + SM_BM - 1) / SM_BM) * ((a.N + 127) / 128);
      if (epi == EPI_GELU)
        hipLaunchKernelGGL((gemm_bf16_mfma_m64<EPI_GELU, true, 128>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_bf16_mfma_m64<EPI_RESID, true, 128>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
      return hipGetLastError();
    }
    const int tiles = a.G * ((a.M + SM_BM - 1) / SM_BM) * ((a.N + BN - 1) / BN);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_m64<EPI_GELU, PK>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    else if (epi == EPI_BIAS && !PK)
      hipLaunchKernelGGL((gemm_bf16_mfma_m64<EPI_BIAS, false>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_m64<EPI_RESID, PK>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  const TileShape shape = PK && (epi == EPI_GELU || epi == EPI_RESID) ? pick_tiles(a, epi) : TILES_256;
  if (shape == TILES_256x384w8) {
    const int tiles6 = a.G * ((a.M + BM - 1) / BM) * (a.N / BN6);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_w8<EPI_GELU>), dim3(tiles6), dim3(W8_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_w8<EPI_RESID>), dim3(tiles6), dim3(W8_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  if (shape == TILES_256x192) {
    const int tiles3 = a.G * ((a.M + BM - 1) / BM) * (a.N / BN3);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_n192<EPI_GELU, 256>), dim3(tiles3), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_n192<EPI_RESID, 256>), dim3(tiles3), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  if (shape == TILES_128x192) {
    const int tiles3 = a.G * ((a.M + 127) / 128) * (a.N / BN3);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_n192<EPI_GELU, 128>), dim3(tiles3), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_n192<EPI_RESID, 128>), dim3(tiles3), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  if (shape == TILES_256x384) {
    const int tiles6 = a.G * ((a.M + BM - 1) / BM) * (a.N / BN6);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_n384<EPI_GELU, 256>), dim3(tiles6), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_n384<EPI_RESID, 256>), dim3(tiles6), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  if (shape == TILES_128x384) {
    const int tilesh = a.G * ((a.M + 127) / 128) * (a.N / BN6);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm_bf16_mfma_n384<EPI_GELU, 128>), dim3(tilesh), dim3(MFMA_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_bf16_mfma_n384<EPI_RESID, 128>), dim3(tilesh), dim3(MFMA_THREADS), 0, stream, a);
    return hipGetLastError();
  }
  const int tiles = a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (epi == EPI_GELU)
    hipLaunchKernelGGL((gemm_bf16_mfma<EPI_GELU, PK>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
  else if (epi == EPI_BIAS && !PK)
    hipLaunchKernelGGL((gemm_bf16_mfma<EPI_BIAS, false>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_bf16_mfma<EPI_RESID, PK>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
  return hipGetLastError();
}

// W [G][K][N] -> W^T packed [G][pk_rows(N) x K]: one thread per 16-byte chunk of the output
// (8 consecutive k of one output row n), padding rows zero.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16_t* __restrict__ W, bf16_t* __restrict__ out,
                                                           int G, int K, int N) {
  const int64_t rows = pk_rows(N);
  const int64_t chunks = int64_t(G) * rows * (K / 8);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks; i += int64_t(gridDim.x) * blockDim.x) {
    const int kc = int(i % (K / 8));
    const int64_t gr = i / (K / 8);
    const int n = int(gr % rows);
    const int g = int(gr / rows);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = n < N ? load1(W + (size_t(g) * K + size_t(kc) * 8 + e) * N + n) : 0.f;
    store8(out + size_t(g) * size_t(rows) * K + pk_off(n, kc * 8, K), v);
  }
}

}  // namespace

hipError_t launch_pack_weights(const void* W, void* out, int G, int K, int N, hipStream_t stream) {
  if (G == 0 || N == 0) return hipSuccess;
  const int64_t chunks = int64_t(G) * pk_rows(N) * (K / 8);
  const int64_t want = (chunks + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(unsigned(want < 65536 ? want : 65536)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(W), static_cast<bf16_t*>(out), G, K, N);
  return hipGetLastError();
}

namespace {

template <typename T>
hipError_t launch_generic(int epi, const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((a.N + GT - 1) / GT, (a.M + GT - 1) / GT, a.G);
  switch (epi) {
    case EPI_GELU: hipLaunchKernelGGL((gemm_generic<T, EPI_GELU>), grid, dim3(256), 0, stream, a); break;
    case EPI_BIAS: hipLaunchKernelGGL((gemm_generic<T, EPI_BIAS>), grid, dim3(256), 0, stream, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_generic<T, EPI_RESID>), grid, dim3(256), 0, stream, a); break;
    case EPI_GELU_SAVE: hipLaunchKernelGGL((gemm_generic<T, EPI_GELU_SAVE>), grid, dim3(256), 0, stream, a); break;
    case EPI_GELU_BWD: hipLaunchKernelGGL((gemm_generic<T, EPI_GELU_BWD>), grid, dim3(256), 0, stream, a); break;
    case EPI_RESID32: hipLaunchKernelGGL((gemm_generic<T, EPI_RESID32>), grid, dim3(256), 0, stream, a); break;
    case EPI_STORE32: hipLaunchKernelGGL((gemm_generic<T, EPI_STORE32>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The backward products and the training forward's GELU epilogue: 256 x 256 tiles only.
template <bool AT, bool BT>
hipError_t launch_dense_mfma_t(int epi, const GemmArgs& a, hipStream_t stream) {
  const dim3 tiles(unsigned(a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN)));
  switch (epi) {
    case EPI_GELU_BWD:
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_GELU_BWD, false, AT, BT>), tiles, dim3(MFMA_THREADS), 0, stream, a);
      break;
    case EPI_RESID32:
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_RESID32, false, AT, BT>), tiles, dim3(MFMA_THREADS), 0, stream, a);
      break;
    case EPI_STORE32:
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_STORE32, false, AT, BT>), tiles, dim3(MFMA_THREADS), 0, stream, a);
      break;
    case EPI_GELU_SAVE:
      if (AT || BT) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_bf16_mfma<EPI_GELU_SAVE, false, false, false>), tiles, dim3(MFMA_THREADS), 0,
                         stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

namespace {

GemmArgs normalized(const GemmArgs& args) {
  GemmArgs a = args;
  if (a.lda == 0) a.lda = a.at ? a.M : a.K;
  if (a.ldc == 0) a.ldc = a.N;
  if (a.sa == 0) a.sa = a.at ? int64_t(a.K) * a.lda : int64_t(a.M) * a.lda;
  if (a.sc == 0) a.sc = int64_t(a.M) * a.ldc;
  return a;
}

}  // namespace

bool gemm_writes_colsum(int dtype, int epi, const GemmArgs& args) {
  const GemmArgs a = normalized(args);
  return (epi == EPI_GELU_BWD || epi == EPI_RESID32) && !a.packed &&
         gemm_uses_mfma(dtype, a.M, a.N, a.K, a.lda, a.at, a.bt) && (a.sa % 8) == 0;
}

namespace {

// W [G][K][N] -> W^T [G][pk_rows(N) x K] in MXFP8: one thread per (output row n, 32-value
// block of K), n fastest so that the reads of W rows coalesce; padding rows zero.
__global__ __launch_bounds__(256) void pack_weights_mx_kernel(const bf16_t* __restrict__ W, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int G, int K, int N) {
  const int64_t rows = pk_rows(N), nkb = K / 32;
  const int64_t total = int64_t(G) * rows * nkb;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int n = int(i % rows);
    const int64_t rest = i / rows;
    const int kb = int(rest % nkb);
    const int g = int(rest / nkb);
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      v[j] = n < N ? load1(W + (size_t(g) * K + size_t(kb) * 32 + j) * N + n) : 0.f;
      amax = fmaxf(amax, fabsf(v[j]));
    }
    const uint32_t sb = mx_scale_bits(amax);
    const float inv = mx_inv_scale(sb);
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] *= inv;
    uint8_t* cg = codes + size_t(g) * size_t(rows) * K;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint2*>(cg + mx_off(n, kb * 32 + 16 * (c >> 1), K) + (c & 1) * 8) = e4m3_pack8(v + 8 * c);
    scales[size_t(g) * size_t(rows) * K / 32 + mx_scale_off(n, kb, K)] = uint8_t(sb);
  }
}

}  // namespace

hipError_t launch_pack_weights_mx(const void* W, void* codes, void* scales, int G, int K, int N, hipStream_t stream) {
  if (G == 0 || N == 0) return hipSuccess;
  if (K % MX_BK) return hipErrorInvalidValue;
  const int64_t total = int64_t(G) * pk_rows(N) * (K / 32);
  const int64_t want = (total + 255) / 256;
  hipLaunchKernelGGL(pack_weights_mx_kernel, dim3(unsigned(want < 65536 ? want : 65536)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(W), static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), G, K,
                     N);
  return hipGetLastError();
}

bool gemm_mx_supported(int M, int N, int K) {
  return M > 0 && N > 0 && K >= MX_BK && K % MX_BK == 0 && N % 32 == 0 &&
         uint64_t(K) * MX_CODE_BYTES / MX_BK < (uint64_t(1) << 31);
}

hipError_t launch_gemm_mx(int epi, const GemmArgs& args, hipStream_t stream) {
  if (args.G == 0 || args.M == 0 || args.N == 0) return hipSuccess;
  if (!gemm_mx_supported(args.M, args.N, args.K)) return hipErrorInvalidValue;
  GemmArgs a = args;  // the fp32 output of EPI_RESID is row-major [G, M, N]
  if (a.ldc == 0) a.ldc = a.N;
  if (a.sc == 0) a.sc = int64_t(a.M) * a.ldc;
  const dim3 tiles(unsigned(a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN)));
  if (epi == EPI_GELU_MX)
    hipLaunchKernelGGL((gemm_mx_mfma<EPI_GELU_MX>), tiles, dim3(MFMA_THREADS), 0, stream, a);
  else if (epi == EPI_RESID)
    hipLaunchKernelGGL((gemm_mx_mfma<EPI_RESID>), tiles, dim3(MFMA_THREADS), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& args, hipStream_t stream) {
  if (args.G == 0 || args.M == 0 || args.N == 0) return hipSuccess;
  GemmArgs a = normalized(args);
  const bool bwd_epi = epi == EPI_GELU_BWD || epi == EPI_RESID32 || epi == EPI_STORE32;
  if ((a.at || a.bt) && !bwd_epi) return hipErrorInvalidValue;
  if (a.packed == GEMM_PACKED_W) {
    // prepared W^T with row-major A and outputs: the training forward's products
    if (dtype != DT_BF16 || (epi != EPI_GELU_SAVE && epi != EPI_RESID) || !gemm_packed_w_supported(a.M, a.N, a.K) ||
        a.lda != a.K || a.ldc != a.N || a.sa != int64_t(a.M) * a.K || a.sc != int64_t(a.M) * a.N)
      return hipErrorInvalidValue;
    const int tiles = a.G * ((a.M + BM - 1) / BM) * (a.N / BN6);
    if (four_wave_tiles()) {
      if (epi == EPI_GELU_SAVE)
        hipLaunchKernelGGL((gemm_bf16_mfma_n384g<EPI_GELU_SAVE>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_bf16_mfma_n384g<EPI_RESID>), dim3(tiles), dim3(MFMA_THREADS), 0, stream, a);
    } else if (epi == EPI_GELU_SAVE) {
      hipLaunchKernelGGL((gemm_bf16_mfma_w8g<EPI_GELU_SAVE>), dim3(tiles), dim3(W8_THREADS), 0, stream, a);
    } else {
      hipLaunchKernelGGL((gemm_bf16_mfma_w8g<EPI_RESID>), dim3(tiles), dim3(W8_THREADS), 0, stream, a);
    }
    return hipGetLastError();
  }
  if (a.packed) {
    // packed operands exist only for the MFMA kernels, and only for the inference epilogues
    if (!gemm_uses_mfma(dtype, a.M, a.N, a.K) || (epi != EPI_GELU && epi != EPI_RESID)) return hipErrorInvalidValue;
    return launch_dense_mfma<true>(epi, a, stream);
  }
  if (gemm_uses_mfma(dtype, a.M, a.N, a.K, a.lda, a.at, a.bt) && (a.sa % 8) == 0) {
    if (a.at) return launch_dense_mfma_t<true, false>(epi, a, stream);
    if (a.bt) return launch_dense_mfma_t<false, true>(epi, a, stream);
    if (bwd_epi || epi == EPI_GELU_SAVE) return launch_dense_mfma_t<false, false>(epi, a, stream);
    return launch_dense_mfma<false>(epi, a, stream);
  }
  return dtype == DT_BF16 ? launch_generic<bf16_t>(epi, a, stream) : launch_generic<float>(epi, a, stream);
}

}  // namespace rmx
