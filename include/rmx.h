/*
 * rmx.h -- C ABI of the MI355X (gfx950) RankMixer block forward library (librmx.so).
 *
 * What it computes.  For a batch of feature-token matrices X[B, T, D] and L blocks,
 * each block n = 1..L does (pages cited by title and section):
 *   S   = LN1(TokenMixing(X) + X)          "RankMixer: Scaling Up Ranking Models in
 *   X'  = LN2(PFFN(S) + S)                  Industrial Recommenders" (translation),
 *                                           section 3.1 eq (1) and 3.3.1 eq (5)
 *   TokenMixing with H = T heads:  M[h, t*q + r] = X[t, h*q + r],  q = D / T
 *                                           (same paper, section 3.3.1 eq (3)-(4);
 *                                           "RankMixer 详解（1）", section 3.1)
 *   PFFN: token t has its own FFN,  v_t = GELU(s_t W1[t] + b1[t]) W2[t] + b2[t],
 *         GELU exact (u * Phi(u))       (paper section 3.3.2 eq (6)-(9);
 *                                        "RankMixer 详解（1）", section 4.1)
 *   Sparse-MoE PFFN (optional): v_t = sum_e g_e * expert_e(s_t), g = ReLU(s_t Wg[t])
 *                                       (paper section 3.4 eq (10))
 *   LN: per row over D, biased variance, eps inside the square root, one gamma/beta
 *       of length D per LayerNorm shared by the T rows ("RankMixer 详解（1）", 3.3)
 * and the output is the mean over tokens of X_L: out[b, :] = (1/T) sum_t X_L[b, t, :]
 * (paper section 3.1; "RankMixer 详解（1）", section 5.1).
 *
 * Conventions shared by every entry point.
 *   - Pointers named as device pointers must point to device memory of the current
 *     HIP device (hipMalloc'd, or torch CUDA tensors on ROCm); every such pointer must
 *     be 16-byte aligned.  All arrays are dense, row-major, last index fastest.
 *   - The caller owns every buffer it passes, and the stream.  The library keeps no
 *     caller pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *     call returns without synchronising.  Outputs are overwritten, never accumulated.
 *   - Errors: every argument and shape check runs on the host before anything is
 *     enqueued; on any error nothing is enqueued and the outputs are untouched.
 *     A failed launch returns RMX_ERR_HIP.  A fault during execution surfaces at the
 *     caller's next synchronisation of the stream.  rmx_last_error() gives the detail.
 *   - A handle may be used by one stream at a time; distinct handles are independent.
 */
#ifndef RMX_H
#define RMX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMX_ABI_VERSION 6

typedef struct rmx_handle rmx_handle; /* opaque, owned by the library */

typedef enum {
  RMX_OK = 0,
  RMX_ERR_INVALID_ARG = 1,   /* a null/misaligned/host pointer, a shape or size mismatch */
  RMX_ERR_UNSUPPORTED = 2,   /* valid but not supported here: device not gfx950, a size limit */
  RMX_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed in rmx_create */
  RMX_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} rmx_status;

typedef enum { RMX_FP32 = 0, RMX_BF16 = 1 } rmx_dtype;

/* How the tokens of a sample exchange information before LN1. */
typedef enum {
  RMX_ROUTING_MIX = 0,       /* Token Mixing (the RankMixer block) */
  RMX_ROUTING_ATTENTION = 1  /* self-attention between the tokens: the comparator of the pages' routing ablation */
} rmx_routing;

/* Model configuration, fixed for the life of a handle.
 *   T, D     tokens per sample and width; H = T always, D % T == 0 required
 *            (paper section 3.3.1: H = T keeps the token count for the residual).
 *   k        FFN expansion: the hidden width is k*D (paper section 3.3.2 eq (7)).
 *   L        number of stacked blocks (paper section 3.1 eq (1)), L >= 1.
 *   dtype    storage and MFMA input type of X, every weight, S and the hidden
 *            activations (and of the Sparse-MoE PFFN's gate-scaled expert outputs, which
 *            the combine sums in fp32).  Accumulation, LayerNorm and GELU are always fp32;
 *            the dense block's pre-LN2 rows stay fp32.
 *   ln_eps   LayerNorm epsilon (1e-5 in "RankMixer 详解（1）", section 6.1).
 *   max_batch  largest B a forward call may pass; the workspace is sized for it.
 *   moe_experts  0 = dense per-token FFN; E > 0 = Sparse-MoE PFFN with E experts per
 *            token (paper section 3.4 eq (10)); moe_hidden = hidden width of one expert.
 *   routing  rmx_routing.  RMX_ROUTING_ATTENTION replaces TokenMixing(X) in every block by
 *            single-head self-attention between the sample's tokens,
 *            softmax(Q K^T / sqrt(D)) V with Q = X Wq, K = X Wk, V = X Wv (D x D projections
 *            shared by the tokens, no output projection): the comparator of the paper's
 *            routing ablation (section 4.4; attention as "RankMixer 详解（1）" section 3.4
 *            writes it).  Dense handles with T <= 64; forward only (no prepared weights,
 *            no training).
 * Limits: dtype BF16 needs D % 8 == 0 and (D/T) % 8 == 0, dtype FP32 needs nothing
 * more; D <= 4096; T*D*sizeof(dtype) <= 96 KiB (one sample must fit the on-chip LDS
 * of one workgroup).  Beyond a limit rmx_create returns RMX_ERR_UNSUPPORTED. */
typedef struct {
  int32_t T;
  int32_t D;
  int32_t k;
  int32_t L;
  int32_t dtype;      /* rmx_dtype */
  float ln_eps;
  int64_t max_batch;
  int32_t moe_experts;
  int32_t moe_hidden;
  int32_t routing;    /* rmx_routing */
} rmx_config;

/* Device pointers to the parameters of all L blocks, each stacked over L, in the
 * config's dtype.  Row-vector convention x W + b (paper section 3.3.2 eq (7)).
 *   W1 [L, T, D, kD]   b1 [L, T, kD]   (b1 may be NULL: zeros)
 *   W2 [L, T, kD, D]   b2 [L, T, D]    (b2 may be NULL: zeros)
 *   ln1_g, ln1_b, ln2_g, ln2_b  [L, D]  (gamma/beta of the two LayerNorms of a block)
 * Sparse-MoE only (else NULL; W1/b1/W2/b2 are then unused and may be NULL):
 *   Wg  [L, T, D, E]              router weights, no bias
 *   We1 [L, T, E, D, h]  be1 [L, T, E, h]   (be1 may be NULL)
 *   We2 [L, T, E, h, D]  be2 [L, T, E, D]   (be2 may be NULL)
 * packed: NULL, or the weights of all blocks prepared by rmx_pack_weights for this handle:
 *   W1 and W2 (dense bf16 handles whose D and k*D are multiples of 32), or We1 and We2
 *   (Sparse-MoE handles whose D and h are multiples of 384).  When set, the forward reads
 *   those weights from it (W1 and W2, or We1 and We2, are then unused and may be NULL);
 *   the result is the same bit for bit.
 * packed_mxfp8: NULL, or W1 and W2 of all blocks prepared by rmx_pack_weights_mxfp8; when
 *   set (and packed is NULL) the forward runs the MXFP8 inference variant (see there).
 * Wq, Wk, Wv [L, D, D]: the self-attention projections of RMX_ROUTING_ATTENTION handles
 *   (row-vector convention x W), else NULL.                                               */
typedef struct {
  const void* W1;
  const void* b1;
  const void* W2;
  const void* b2;
  const void* ln1_g;
  const void* ln1_b;
  const void* ln2_g;
  const void* ln2_b;
  const void* Wg;
  const void* We1;
  const void* be1;
  const void* We2;
  const void* be2;
  const void* packed;
  const void* packed_mxfp8;
  const void* Wq;
  const void* Wk;
  const void* Wv;
} rmx_weights;

/* Validates cfg, checks that the current HIP device is gfx950, and allocates the
 * workspace for cfg->max_batch samples on it.  On success *out_handle is a new handle;
 * on failure it is set to NULL and nothing stays allocated. */
rmx_status rmx_create(const rmx_config* cfg, rmx_handle** out_handle);

/* Frees the handle and its workspace (synchronises the device first).  NULL is a no-op. */
rmx_status rmx_destroy(rmx_handle* h);

/* The forward pass.  X [B, T, D] (device, dtype) -> out [B, D] (device, fp32), the mean
 * pool of X_L.  L and k must equal the handle's (they are restated so that a caller's
 * mismatch is caught).  0 <= B <= max_batch; B == 0 enqueues nothing and returns OK. */
rmx_status rmx_block_forward(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w,
                             int32_t L, int32_t k, float* out, void* stream);

/* rmx_block_forward plus optional diagnostic outputs (either may be NULL):
 *   xl_out   [B, T, D] (device, dtype)  X_L, the last block's output, rounded to dtype
 *   gate_out [L, B, T, E] (device, fp32) the Sparse-MoE gate values of every block
 *            (MoE handles only; must be NULL for a dense handle). */
rmx_status rmx_block_forward_ex(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w,
                                int32_t L, int32_t k, float* out, void* xl_out,
                                float* gate_out, void* stream);

/* The token -> expert row lists of a Sparse-MoE forward, every block: a diagnostic output
 * (the integer routing step of the paper translation, section 3.4 eq (10): each token
 * activates a variable number of its experts, those whose ReLU gate is positive).  With
 * G = T*E groups, group gi = t*E + e lists the samples b whose gate g[b, t, e] > 0:
 *   group_start [L, G + 1] int32  the list of group gi is rows[group_start[gi] ..
 *                                 group_start[gi + 1]), group_start[0] = 0
 *   rows        [L, G * B] int32  the lists, concatenated in group order; each entry is the
 *                                 token row t*B + b, ascending in b within a group; entries
 *                                 from group_start[G] on are left unspecified
 *   row_gate    [L, G * B] fp32   the gate g[b, t, e] of each listed row (same positions)
 *   pos         [L, G, B]  int32  inverse map: position of (t, e, b) in rows, or -1
 *   tile_start  [L, G + 1] int32  cumulative count of 256-row product tiles over the groups
 * Every member is a device pointer or NULL (not written).  The member arrays for block n
 * start at n times the per-block size given above. */
typedef struct {
  int32_t* group_start;
  int32_t* rows;
  float* row_gate;
  int32_t* pos;
  int32_t* tile_start;
} rmx_moe_lists;

/* rmx_block_forward_ex that also copies the routing lists of every block to `lists`
 * (Sparse-MoE handles only; INVALID_ARG for a dense handle or a NULL `lists`).  The
 * forward's results are those of rmx_block_forward_ex. */
rmx_status rmx_block_forward_moe_lists(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w,
                                       int32_t L, int32_t k, float* out, void* xl_out, float* gate_out,
                                       const rmx_moe_lists* lists, void* stream);

/* Token Mixing alone (H = T): Y[b, h, t*q + r] = X[b, t, h*q + r], q = D/T, for every
 * sample; X and Y are device arrays [B, T, D] of `dtype` and must not overlap.  Uses
 * the same device index map as the forward pass.  Exact: values are copied bit for bit.
 * (Paper section 3.3.1 eq (3)-(4); "RankMixer 详解（1）", section 3.1.) */
rmx_status rmx_token_mix(const void* X, void* Y, int64_t B, int32_t T, int32_t D,
                         int32_t dtype, void* stream);

/* Weights prepared once for the matrix cores.  rmx_packed_weights_bytes gives the size of
 * the prepared copy of W1 and W2 (dense handles) or We1 and We2 (Sparse-MoE handles) of all
 * L blocks for this handle, or 0 when the handle has no such path (fp32; dense with D or
 * k*D not a multiple of 32; Sparse-MoE with D or moe_hidden not a multiple of 384).
 * rmx_pack_weights reads w->W1 and w->W2 (device, [L, T, D, kD] and [L, T, kD, D]), or
 * w->We1 and w->We2 ([L, T, E, D, h] and [L, T, E, h, D]), and writes the copy to `packed`
 * (device, `bytes` >= rmx_packed_weights_bytes(h), 16-byte aligned, not overlapping the
 * sources), enqueued on `stream`: each token's (each expert's) W^T in blocks of 256 rows x
 * 32 columns, so that a K step of a 256-column weight tile is one contiguous 16 KB.  Pass it
 * as rmx_weights.packed.  The caller owns the buffer; it stays valid while the source
 * weights are unchanged.  Errors: INVALID_ARG for a short or overlapping buffer, a wrong L
 * or a pointer off the handle's device; UNSUPPORTED where the size above is 0. */
size_t rmx_packed_weights_bytes(const rmx_handle* h);
rmx_status rmx_pack_weights(rmx_handle* h, const rmx_weights* w, int32_t L, void* packed, size_t bytes,
                            void* stream);
/* Tile shapes of the products on prepared weights are chosen per launch from the device's
 * CU count.  Two environment variables, read at each launch, force them (for tests and
 * tuning; every choice gives the same bits): RMX_WIDE_TILES = always | half | pair | pairhalf |
 * wide8 | never (256 x 384, 128 x 384, 256 x 192 or 128 x 192 with two workgroups per CU,
 * 256 x 384 with eight waves, or 256 x 256 tiles, above 128 rows per token; the 384-wide
 * shapes need N % 384 == 0, the 192-wide ones N % 192 == 0; `always` also keeps the
 * training forward's and the Sparse-MoE products on four-wave instead of eight-wave
 * 256 x 384 tiles) and
 * RMX_NARROW_TILES = always | never (64 x 128 or 64 x 256 tiles up to 128 rows per token).
 * Other values are ignored. */

/* MXFP8 inference variant.  The pages serve the model at reduced precision because its
 * core is a few large products and halving the operand width doubles the hardware peak
 * ("RankMixer" paper translation, section 4.6, eq (13)); on gfx950 the step beyond bf16 is
 * 8-bit operands.  The operands of both per-token products are stored in MXFP8 as the OCP
 * Microscaling Formats (MX) Specification v1.0 defines it: FP8 E4M3 codes, one power-of-two
 * scale 2^(floor(log2 amax) - 8) per 32 consecutive values along K, each value rounded to the
 * nearest E4M3 number (ties to even, saturating at +-448).  Quantized: S along D per row, H
 * = GELU(S W1 + b1) along kD per row, W1[t] and W2[t] along K per output column.  Products
 * accumulate in fp32 on the matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4); bias, GELU,
 * residual (S in bf16), LayerNorm and pool as in the bf16 forward.  Expect about 4e-2
 * relative difference from the unquantized forward (the format's precision).
 * rmx_packed_weights_mxfp8_bytes: bytes of W1 and W2 of all L blocks in this form, or 0 when
 * the handle has no such path (it needs a dense bf16 handle with D and k*D multiples of 64).
 * rmx_pack_weights_mxfp8: reads w->W1 and w->W2 (device, bf16) and writes them to `packed`
 * (device, `bytes` >= the size above, 16-byte aligned), enqueued on `stream`; pass it as
 * rmx_weights.packed_mxfp8. */
size_t rmx_packed_weights_mxfp8_bytes(const rmx_handle* h);
rmx_status rmx_pack_weights_mxfp8(rmx_handle* h, const rmx_weights* w, int32_t L, void* packed, size_t bytes,
                                  void* stream);

/* Tokenisation projection, the step before the first block: the concatenated feature
 * embedding E [B, T*d] (device, dtype) is cut into T half-open slices of d coordinates and
 * slice t is projected by token t's own layer,
 *     X[b, t, :] = E[b, t*d : (t+1)*d] Wp[t] + bp[t],
 * Wp [T, d, D] (device, dtype, row-vector convention), bp [T, D] (device, dtype, or NULL =
 * zeros), X [B, T, D] (device, dtype): the input of rmx_block_forward.  E and X must not
 * overlap.  fp32 or bf16; the products accumulate in fp32 and X is rounded to dtype.
 * T, d, D >= 1, B >= 0 (B == 0 enqueues nothing).  Stateless: no handle.
 * ("RankMixer" paper translation, section 3.2 eq (2); "RankMixer 详解（1）", section 2;
 * "UniMixer" translation, eq (9) for the token-specific layers.) */
rmx_status rmx_tokenize(const void* E, const void* Wp, const void* bp, void* X, int64_t B, int32_t T,
                        int32_t d, int32_t D, int32_t dtype, void* stream);

/* Training: the forward pass that keeps the activations the backward pass needs, and the
 * backward pass ("RankMixer 详解（1）：特征分组与完整计算流程", section 5.2).  Dense handles
 * (moe_experts == 0) only.  Both calls need W1 and W2.  rmx_block_forward_train may also be
 * given w->packed (rmx_pack_weights for this handle): its products then read W1 and W2 from
 * the prepared copy where their shapes allow (N a multiple of 384), with the same results
 * bit for bit; rmx_block_backward reads W1 and W2 and ignores w->packed.
 *
 * rmx_saved_bytes: bytes of the saved activations for B samples (0 for a Sparse-MoE handle,
 * a NULL handle or B < 0).  Per block: S [T, B, D] (dtype); GELU'(U) at the
 * pre-activations U = S W1 + b1, and the hidden H = GELU(U), [T, B, kD] each (dtype); the
 * pre-LN2 rows [T, B, D] (fp32); each padded to 256 bytes.
 *
 * rmx_block_forward_train: rmx_block_forward (same out, bit for bit) that also writes the
 * saved activations to `saved` (device, `saved_bytes` >= rmx_saved_bytes(h, B)).
 *
 * rmx_block_backward: given g_out [B, D] (device, fp32), the gradient of a loss with respect
 * to out, writes the gradient of that loss with respect to X, dX [B, T, D] (device, fp32),
 * and with respect to every parameter, summed over the B samples (scale g_out by 1/B for a
 * mean loss), into `grads` (device, fp32, all required, shaped like the weights):
 *   dW1 [L, T, D, kD]  db1 [L, T, kD]  dW2 [L, T, kD, D]  db2 [L, T, D]
 *   dln1_g, dln1_b, dln2_g, dln2_b [L, D]
 * X, B, w and `saved` must be those of the rmx_block_forward_train call that filled
 * `saved`, which stays unchanged.  The gradients of the pooled output pass through the
 * mean pool, then for each block from the last: LayerNorm backward, the per-token FFN
 * backward (GELU'(u) = Phi(u) + u phi(u)), the second residual, LayerNorm backward, and
 * the first residual with the mixing transpose, dX = (P^T + I) g.  Products run on the
 * matrix cores for bf16 (operands rounded to bf16: the gradients of the pre-LN2 rows and of
 * the pre-activations), accumulate in fp32; everything else is fp32.
 * The first backward call on a handle allocates its backward workspace (for max_batch
 * samples; RMX_ERR_OUT_OF_MEMORY if that fails).  Outputs must not overlap the inputs
 * or each other.  Limits: D <= 2048 when D % 8 == 0 and (D/T) % 8 == 0, else D <= 512;
 * T*D*sizeof(dtype) <= 96 KiB.  B == 0 enqueues nothing. */
typedef struct {
  float* dW1;
  float* db1;
  float* dW2;
  float* db2;
  float* dln1_g;
  float* dln1_b;
  float* dln2_g;
  float* dln2_b;
} rmx_grads;

size_t rmx_saved_bytes(const rmx_handle* h, int64_t B);
rmx_status rmx_block_forward_train(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                                   int32_t k, float* out, void* saved, size_t saved_bytes, void* stream);
rmx_status rmx_block_backward(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                              int32_t k, const void* saved, size_t saved_bytes, const float* g_out, float* dX,
                              const rmx_grads* grads, void* stream);

/* Kernel-level timing.  While enabled, every kernel the handle launches is bracketed by
 * a pair of HIP events recorded on the caller's stream; rmx_profile_read() waits for the
 * recorded events and returns, per kernel kind, the summed duration in ms and the
 * number of launches since the last reset.  Up to 65536 launches are kept between
 * reads; later ones are counted in `dropped` and not timed. */
typedef enum {
  RMX_KERNEL_ROWS = 0,     /* LN2 of the previous block (if any) + mixing + residual + LN1 */
  RMX_KERNEL_GEMM1 = 1,    /* per-token S W1 + b1, GELU -> hidden */
  RMX_KERNEL_GEMM2 = 2,    /* per-token hidden W2 + b2 + S -> pre-LN2 rows */
  RMX_KERNEL_POOL = 3,     /* LN2 of the last block + mean pool (+ X_L) */
  RMX_KERNEL_MOE_GATE = 4, /* router + token -> expert lists */
  RMX_KERNEL_MOE_FFN1 = 5, /* expert first layer (gathered rows) + GELU */
  RMX_KERNEL_MOE_FFN2 = 6, /* expert second layer, gate-weighted */
  RMX_KERNEL_MOE_COMBINE = 7, /* not launched: the sum of the expert rows + S is formed in the
                                 next row pass (RMX_KERNEL_ROWS / RMX_KERNEL_POOL) */
  RMX_KERNEL_BWD_ROWS = 8, /* backward: LayerNorm backward, mixing transpose, residuals */
  RMX_KERNEL_BWD_DU = 9,   /* backward: per-token gY W2^T * GELU'(U) -> gU */
  RMX_KERNEL_BWD_DS = 10,  /* backward: per-token gU W1^T + gY -> gradient of S */
  RMX_KERNEL_BWD_DW1 = 11, /* backward: per-token S^T gU -> dW1 */
  RMX_KERNEL_BWD_DW2 = 12, /* backward: per-token H^T gY -> dW2 */
  RMX_KERNEL_BWD_SUMS = 13, /* backward: batch sums of the bias and LayerNorm gradients */
  RMX_KERNEL_ATTN_QKV = 14, /* attention routing: the Q, K, V projections */
  RMX_KERNEL_ATTN = 15,     /* attention routing: softmax(Q K^T / sqrt(D)) V + X, LN1 */
  RMX_KERNEL_COUNT = 16
} rmx_kernel_kind;

rmx_status rmx_profile_enable(rmx_handle* h, int32_t enable);
rmx_status rmx_profile_read(rmx_handle* h, double* total_ms /*[RMX_KERNEL_COUNT]*/,
                            int64_t* launches /*[RMX_KERNEL_COUNT]*/, int64_t* dropped);
rmx_status rmx_profile_reset(rmx_handle* h);
const char* rmx_kernel_name(int32_t kind);

/* Short text for a status code; never NULL. */
const char* rmx_status_string(rmx_status s);

/* Detail of the last failure: of this handle's last call when h != NULL, else of the
 * calling thread's last call (rmx_create, rmx_token_mix, rmx_tokenize).  Never NULL; "" if
 * none. */
const char* rmx_last_error(const rmx_handle* h);

/* Forward pass that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It is rmx_block_forward for a dense Token Mixing configuration (moe_experts == 0,
 * routing == RMX_ROUTING_MIX), with no handle: `cfg` is validated as rmx_create would
 * (max_batch is ignored), and `w` holds W1/W2 or `packed` from rmx_pack_weights (on a
 * handle of the same configuration; packed_mxfp8 is refused).  The results are those of
 * rmx_block_forward with the same arguments, bit for bit.
 * Workspace: the library keeps one array of RMX_NOALLOC_SCRATCH_BYTES of device memory per
 * device it runs on (held from the first use on that device until the process ends) and
 * lays the workspace of a handle with max_batch = B into it:
 *   round256(P*D*s) + round256(P*k*D*s) + T*B*D*4 bytes,  s = sizeof(dtype),
 *   P = T * (B rounded up to a multiple of 256) for bf16 configurations with D and k*D
 *   multiples of 32, else P = T * B.
 * Beyond the limit the call returns RMX_ERR_UNSUPPORTED (at the RankMixer-1B shape,
 * T=32, D=1536, k=4, bf16: B <= 256; at T=16, D=768, k=4: B <= 1024).  Every call on one
 * device uses that device's array, so calls on one device whose executions overlap (on
 * different streams, or from different threads) race and must be ordered by the caller.
 * The first call on a device sets the device up (architecture check, the array's address);
 * no call allocates device memory.  Errors as rmx_block_forward; the detail is in
 * rmx_last_error(NULL). */
#define RMX_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
rmx_status rmx_block_forward_noalloc(const rmx_config* cfg, const void* X, int64_t B, const rmx_weights* w,
                                     float* out, void* stream);

/* RMX_ABI_VERSION of the built library. */
int32_t rmx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RMX_H */
