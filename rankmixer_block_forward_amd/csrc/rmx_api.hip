// C ABI of the RankMixer block forward (declared in include/rmx.h): handle and workspace,
// argument checks, the launch sequence of one forward pass, and kernel timing.
//
// Launch sequence for L blocks (all on the caller's stream):
//   n = 1..L:  rows   (LN2 of block n-1, or X0 for n = 1; mixing; residual; LN1) -> S
//              gemm1  S[t] W1[t] + b1[t], GELU                                   -> H
//              gemm2  H[t] W2[t] + b2[t] + S[t]                                   -> Y
//   then:      rows   LN2 of block L, mean pool over tokens (+ X_L)              -> out
// With the Sparse-MoE PFFN (moe_experts > 0) gemm1 / gemm2 are replaced by: route (gate,
// scan, scatter), the grouped expert GEMMs over the compacted row lists, and combine.
// (RankMixer paper translation, section 3.1 eq (1) and 3.3; "RankMixer 详解（1）",
// sections 3-5.)  Workspace, all token-major [T, max_batch, *]: S and H in the model
// dtype, Y in fp32.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <new>
#include <type_traits>
#include <string>
#include <vector>

#include "../../include/rmx.h"
#include "rmx_internal.h"

using namespace rmx;

namespace {

thread_local std::string g_thread_error;

struct ProfPair {
  int kind;
  hipEvent_t start, stop;
};

constexpr size_t PROF_CAP = 65536;

}  // namespace

struct rmx_handle {
  rmx_config cfg{};
  int device = -1;
  void* S = nullptr;   // [T, max_batch, D]   dtype
  void* H = nullptr;   // [T, max_batch, kD]  dtype
  float* Y = nullptr;  // [T, max_batch, D]   fp32
  // Dense bf16 handles with D and kD multiples of 32 can run on prepared weights; S and H
  // then take the packed operand layout and are sized for pk_rows(max_batch) rows.
  bool pk_capable = false;
  // pk_capable handles with D and kD multiples of 64 also run the MXFP8 variant: S in MXFP8
  // (codes [T, pk_rows(max_batch), D] bytes, then their scales, 1/32 of that), and H in
  // MXFP8 in the H buffer (codes, then scales)
  bool mx_capable = false;
  // Sparse-MoE bf16 handles with D and moe_hidden multiples of 384 can run their expert
  // products on prepared expert weights (each expert's W^T packed, 256 x 384 tiles)
  bool moe_pk_capable = false;
  void* S8 = nullptr;
  // Sparse-MoE workspace (moe_experts > 0); G = T * E groups, R = G * max_batch rows
  float* moe_g = nullptr;        // [G, max_batch]
  int* moe_cnt = nullptr;        // [G, nchunk]
  int* moe_chunk_off = nullptr;  // [G, nchunk]
  int* moe_group_rows = nullptr; // [G]
  int* moe_group_start = nullptr;// [G + 1]
  int* moe_tile_start = nullptr; // [G + 1]
  int* moe_src_row = nullptr;    // [R]
  float* moe_row_gate = nullptr; // [R]
  int* moe_pos = nullptr;        // [G, max_batch]
  void* moe_hidden = nullptr;    // [R, h] bf16, or packed on tile-aligned group blocks
  void* moe_out = nullptr;       // [R, D]  bf16 gate-scaled expert rows
  // Self-attention routing (routing == RMX_ROUTING_ATTENTION): Q, K, V and the block input
  // of blocks 2..L, each [max_batch, T, D] dtype, and a scratch for the unused pool of the
  // launch that forms that input
  void* aQ = nullptr;
  void* aK = nullptr;
  void* aV = nullptr;
  void* aX = nullptr;
  float* a_pool = nullptr;       // [max_batch, D]
  // Backward workspace, allocated by the first backward call (all for max_batch samples)
  bool bwd_ready = false;
  float* bw_gY32 = nullptr;      // [T, max_batch, D]  fp32  gradient of the pre-LN2 rows
  void* bw_gY = nullptr;         // [T, max_batch, D]  dtype the same, a GEMM operand
  void* bw_gU = nullptr;         // [T, max_batch, kD] dtype gradient of the pre-activations
  float* bw_gS = nullptr;        // [T, max_batch, D]  fp32  gradient of S
  float* bw_gR = nullptr;        // [max_batch, T, D]  fp32  row-kernel scratch
  float* bw_part1 = nullptr;     // [2, max_batch, D]  fp32  per-sample LN1 gamma / beta gradients
  float* bw_part2 = nullptr;     // [2, max_batch, D]  fp32  per-sample LN2 gamma / beta gradients
  float* bw_sum = nullptr;       // column-sum scratch
  float* bw_cpart = nullptr;     // [T, colsum_rows(max_batch), max(k D, D)] per-wave column sums
  std::vector<void*> allocs;     // everything hipMalloc'd, freed by rmx_destroy
  std::string last_error;
  bool prof = false;
  std::vector<ProfPair> pending;
  std::vector<hipEvent_t> free_events;
  double total_ms[RMX_KERNEL_COUNT] = {};
  int64_t launches[RMX_KERNEL_COUNT] = {};
  int64_t dropped = 0;
};

namespace {

rmx_status fail(rmx_handle* h, rmx_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (h)
    h->last_error = buf;
  else
    g_thread_error = buf;
  return s;
}

void clear_error(rmx_handle* h) {
  if (h)
    h->last_error.clear();
  else
    g_thread_error.clear();
}

// A device pointer is acceptable when it is 16-byte aligned and the bytes
// [p, p + bytes) lie inside one allocation of `device`.
rmx_status check_dev(rmx_handle* h, const void* p, size_t bytes, int device, const char* name) {
  if (!p) return fail(h, RMX_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(h, RMX_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "%s is not a HIP allocation", name);
  }
  if (attr.type != hipMemoryTypeDevice)
    return fail(h, RMX_ERR_INVALID_ARG, "%s is not device memory", name);
  if (attr.device != device)
    return fail(h, RMX_ERR_INVALID_ARG, "%s lives on device %d, not %d", name, attr.device, device);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "%s: allocation range unknown", name);
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  if (q + bytes > b + size)
    return fail(h, RMX_ERR_INVALID_ARG, "%s: %zu bytes needed but only %zu remain in its allocation",
                name, bytes, size_t(b + size - q));
  return RMX_OK;
}

rmx_status check_dev_opt(rmx_handle* h, const void* p, size_t bytes, int device, const char* name) {
  return p ? check_dev(h, p, bytes, device, name) : RMX_OK;
}

rmx_status check_device_arch(rmx_handle* h, int* device_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_UNSUPPORTED, "no HIP device");
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_HIP, "hipGetDeviceProperties failed");
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(h, RMX_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                prop.gcnArchName);
  *device_out = dev;
  return RMX_OK;
}

rmx_status validate_config(const rmx_config* c) {
  if (!c) return fail(nullptr, RMX_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 1 || c->D < 1 || c->k < 1 || c->L < 1)
    return fail(nullptr, RMX_ERR_INVALID_ARG, "T, D, k, L must all be >= 1 (got %d, %d, %d, %d)", c->T,
                c->D, c->k, c->L);
  if (c->D % c->T)
    return fail(nullptr, RMX_ERR_INVALID_ARG, "D=%d is not divisible by H=T=%d", c->D, c->T);
  if (c->dtype != RMX_FP32 && c->dtype != RMX_BF16)
    return fail(nullptr, RMX_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (!(c->ln_eps > 0.f)) return fail(nullptr, RMX_ERR_INVALID_ARG, "ln_eps must be > 0");
  if (c->max_batch < 0) return fail(nullptr, RMX_ERR_INVALID_ARG, "max_batch < 0");
  if (c->moe_experts < 0 || c->moe_hidden < 0)
    return fail(nullptr, RMX_ERR_INVALID_ARG, "moe_experts, moe_hidden must be >= 0");
  if (c->moe_experts > 0) {
    const int E = c->moe_experts, h = c->moe_hidden;
    if (c->dtype != RMX_BF16) return fail(nullptr, RMX_ERR_UNSUPPORTED, "the Sparse-MoE PFFN runs in bf16 only");
    if (h < 1) return fail(nullptr, RMX_ERR_INVALID_ARG, "moe_hidden must be >= 1 when moe_experts > 0");
    if (E > MOE_MAX_E || int64_t(c->T) * E > MOE_MAX_GROUPS || int64_t(c->D) * E > MOE_MAX_GATE_WEIGHTS)
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "MoE limits: E <= %d, T*E <= %d, D*E <= %d", MOE_MAX_E,
                  MOE_MAX_GROUPS, MOE_MAX_GATE_WEIGHTS);
    if (moe_gate_lds_bytes(c->D, E) > MOE_MAX_GATE_LDS)
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "MoE router weights of one token exceed %zu bytes of LDS",
                  size_t(MOE_MAX_GATE_LDS));
    if (!gemm_moe_supported(h, c->D, int64_t(c->T) * c->max_batch, false) ||
        !gemm_moe_supported(c->D, h, c->max_batch, false))
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "MoE GEMMs need D %% 32 == 0, moe_hidden %% 32 == 0 and slices < 2 GiB");
  }
  if (c->routing != RMX_ROUTING_MIX && c->routing != RMX_ROUTING_ATTENTION)
    return fail(nullptr, RMX_ERR_INVALID_ARG, "unknown routing %d", c->routing);
  if (c->routing == RMX_ROUTING_ATTENTION) {
    if (c->moe_experts > 0)
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "attention routing is built for the dense per-token FFN");
    if (int64_t(c->T) * c->max_batch >= (int64_t(1) << 31))
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "attention routing needs T * max_batch < 2^31");
    if (!attn_supported(c->dtype, c->T, c->D))
      return fail(nullptr, RMX_ERR_UNSUPPORTED, "attention routing needs T <= %d and D <= %d", ATTN_MAX_T,
                  ATTN_MAX_D);
  }
  const bool vec = rows_vectorized(c->T, c->D);
  if (c->dtype == RMX_BF16 && !vec)
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "bf16 needs D %% 8 == 0 and (D/T) %% 8 == 0");
  if (c->D > (vec ? ROWS_MAX_D : ROWS_MAX_D_SCALAR))
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "D=%d exceeds the row kernel limit %d", c->D,
                vec ? ROWS_MAX_D : ROWS_MAX_D_SCALAR);
  if (rows_lds_bytes(c->dtype, c->T, c->D) > ROWS_MAX_LDS)
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "one sample (T*D*%d = %zu bytes) exceeds %zu bytes of LDS",
                dtype_size(c->dtype), rows_lds_bytes(c->dtype, c->T, c->D), ROWS_MAX_LDS);
  const int64_t kD = int64_t(c->k) * c->D;
  const int64_t rows = int64_t(c->T) * c->max_batch;
  if (kD > (int64_t(1) << 30) || c->max_batch > (int64_t(1) << 30) || rows * kD > (int64_t(1) << 46))
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "sizes too large");
  return RMX_OK;
}

// ---- kernel timing
void prof_begin(rmx_handle* h, hipStream_t s, ProfPair* pp, int kind) {
  pp->kind = -1;
  if (!h->prof) return;
  if (h->pending.size() >= PROF_CAP) {
    ++h->dropped;
    return;
  }
  auto take = [&]() {
    hipEvent_t e = nullptr;
    if (!h->free_events.empty()) {
      e = h->free_events.back();
      h->free_events.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      e = nullptr;
    }
    return e;
  };
  pp->start = take();
  pp->stop = take();
  if (!pp->start || !pp->stop) {
    if (pp->start) h->free_events.push_back(pp->start);
    if (pp->stop) h->free_events.push_back(pp->stop);
    ++h->dropped;
    return;
  }
  pp->kind = kind;
  (void)hipEventRecord(pp->start, s);
}

void prof_end(rmx_handle* h, hipStream_t s, ProfPair* pp) {
  if (pp->kind < 0) return;
  (void)hipEventRecord(pp->stop, s);
  h->pending.push_back(*pp);
}

hipError_t run_rows(rmx_handle* h, hipStream_t s, int mode, const RowsArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, mode == ROWS_FINAL ? RMX_KERNEL_POOL : RMX_KERNEL_ROWS);
  hipError_t e = launch_rows(h->cfg.dtype, mode, a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_gemm(rmx_handle* h, hipStream_t s, int epi, const GemmArgs& a, int kind = -1) {
  ProfPair pp;
  if (kind < 0) kind = (epi == EPI_GELU || epi == EPI_GELU_SAVE) ? RMX_KERNEL_GEMM1 : RMX_KERNEL_GEMM2;
  prof_begin(h, s, &pp, kind);
  hipError_t e = launch_gemm(h->cfg.dtype, epi, a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_gemm_mx(rmx_handle* h, hipStream_t s, int epi, const GemmArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, epi == EPI_GELU_MX ? RMX_KERNEL_GEMM1 : RMX_KERNEL_GEMM2);
  hipError_t e = launch_gemm_mx(epi, a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_attn(rmx_handle* h, hipStream_t s, const AttnArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, RMX_KERNEL_ATTN);
  hipError_t e = launch_attn_rows(h->cfg.dtype, a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_rows_bwd(rmx_handle* h, hipStream_t s, int mode, const RowsBwdArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, RMX_KERNEL_BWD_ROWS);
  hipError_t e = launch_rows_bwd(h->cfg.dtype, mode, a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_colsum(rmx_handle* h, hipStream_t s, int dtype, const void* in, float* out, int G, int R, int N) {
  ProfPair pp;
  prof_begin(h, s, &pp, RMX_KERNEL_BWD_SUMS);
  hipError_t e = launch_colsum(dtype, in, out, h->bw_sum, G, R, N, s);
  prof_end(h, s, &pp);
  return e;
}

// Saved activations of one block for B samples (byte offsets, each padded to 256 bytes):
// S, GELU' at the pre-activations (U), the hidden H and the pre-LN2 rows Y.
struct SavedLayout {
  size_t S, U, H, Y, per_block;
};

SavedLayout saved_layout(const rmx_config& c, int64_t B) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t esz = dtype_size(c.dtype), rows = size_t(c.T) * size_t(B), kD = size_t(c.k) * c.D;
  SavedLayout l;
  l.S = 0;
  l.U = up(rows * c.D * esz);
  l.H = l.U + up(rows * kD * esz);
  l.Y = l.H + up(rows * kD * esz);
  l.per_block = l.Y + up(rows * c.D * sizeof(float));
  return l;
}

hipError_t run_moe_route(rmx_handle* h, hipStream_t s, const MoeArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, RMX_KERNEL_MOE_GATE);
  hipError_t e = launch_moe_route(a, s);
  prof_end(h, s, &pp);
  return e;
}

hipError_t run_moe_gemm(rmx_handle* h, hipStream_t s, int epi, const GemmArgs& a) {
  ProfPair pp;
  prof_begin(h, s, &pp, epi == EPI_MOE1 ? RMX_KERNEL_MOE_FFN1 : RMX_KERNEL_MOE_FFN2);
  hipError_t e = launch_gemm_moe(epi, a, s);
  prof_end(h, s, &pp);
  return e;
}

}  // namespace

static void set_capabilities(rmx_handle* h);

extern "C" {

int32_t rmx_abi_version(void) { return RMX_ABI_VERSION; }

const char* rmx_status_string(rmx_status s) {
  switch (s) {
    case RMX_OK: return "ok";
    case RMX_ERR_INVALID_ARG: return "invalid argument";
    case RMX_ERR_UNSUPPORTED: return "unsupported";
    case RMX_ERR_OUT_OF_MEMORY: return "out of memory";
    case RMX_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* rmx_last_error(const rmx_handle* h) { return h ? h->last_error.c_str() : g_thread_error.c_str(); }

const char* rmx_kernel_name(int32_t kind) {
  static const char* names[RMX_KERNEL_COUNT] = {"rows_ln2_mix_ln1", "gemm1_gelu",   "gemm2_residual",
                                                "rows_ln2_pool",    "moe_gate",     "moe_ffn1",
                                                "moe_ffn2",         "moe_combine",  "bwd_rows",
                                                "bwd_gemm_dU",      "bwd_gemm_dS",  "bwd_gemm_dW1",
                                                "bwd_gemm_dW2",     "bwd_sums",     "attn_qkv",
                                                "attn_rows"};
  return (kind >= 0 && kind < RMX_KERNEL_COUNT) ? names[kind] : "unknown";
}

rmx_status rmx_create(const rmx_config* cfg, rmx_handle** out_handle) {
  clear_error(nullptr);
  if (!out_handle) return fail(nullptr, RMX_ERR_INVALID_ARG, "out_handle is NULL");
  *out_handle = nullptr;
  rmx_status st = validate_config(cfg);
  if (st != RMX_OK) return st;
  int dev = -1;
  if ((st = check_device_arch(nullptr, &dev)) != RMX_OK) return st;
  hipError_t e;
  if ((e = rows_init()) != hipSuccess || (e = gemm_init()) != hipSuccess || (e = moe_init()) != hipSuccess ||
      (e = rows_bwd_init()) != hipSuccess)
    return fail(nullptr, RMX_ERR_HIP, "kernel set-up failed: %s", hipGetErrorString(e));

  rmx_handle* h = new (std::nothrow) rmx_handle();
  if (!h) return fail(nullptr, RMX_ERR_OUT_OF_MEMORY, "host allocation failed");
  h->cfg = *cfg;
  h->device = dev;
  const size_t esz = dtype_size(cfg->dtype);
  const size_t rows = size_t(cfg->T) * size_t(cfg->max_batch);
  const size_t nS = rows * cfg->D, nH = rows * size_t(cfg->k) * cfg->D;
  size_t total = 0;
  bool ok = true;
  auto alloc = [&](auto** ptr, size_t bytes) {
    if (!ok || bytes == 0) return;
    void* q = nullptr;
    if (hipMalloc(&q, bytes) != hipSuccess) {
      (void)hipGetLastError();
      ok = false;
      return;
    }
    h->allocs.push_back(q);
    *ptr = static_cast<std::remove_pointer_t<std::remove_reference_t<decltype(*ptr)>>*>(q);
    total += bytes;
  };
  set_capabilities(h);
  const size_t prow = h->pk_capable ? size_t(cfg->T) * size_t(pk_rows(cfg->max_batch)) : rows;
  if (rows > 0) {
    alloc(&h->S, prow * cfg->D * esz);
    if (h->mx_capable) alloc(&h->S8, prow * cfg->D + prow * cfg->D / 32);
    if (cfg->routing == RMX_ROUTING_ATTENTION) {
      alloc(&h->aQ, nS * esz);
      alloc(&h->aK, nS * esz);
      alloc(&h->aV, nS * esz);
      alloc(&h->aX, nS * esz);
      alloc(&h->a_pool, size_t(cfg->max_batch) * cfg->D * sizeof(float));
    }
    if (cfg->moe_experts == 0) {
      alloc(&h->Y, nS * sizeof(float));
      alloc(&h->H, prow * size_t(cfg->k) * cfg->D * esz);
    } else {
      // no Y: the row pass after a Sparse-MoE block forms its pre-LN2 rows from S and the
      // expert rows
      const size_t G = size_t(cfg->T) * cfg->moe_experts, mb = size_t(cfg->max_batch);
      const size_t nchunk = (mb + 63) / 64, R = G * mb;
      alloc(&h->moe_g, G * mb * sizeof(float));
      alloc(&h->moe_cnt, G * nchunk * sizeof(int));
      alloc(&h->moe_chunk_off, G * nchunk * sizeof(int));
      alloc(&h->moe_group_rows, G * sizeof(int));
      alloc(&h->moe_group_start, (G + 1) * sizeof(int));
      alloc(&h->moe_tile_start, (G + 1) * sizeof(int));
      alloc(&h->moe_src_row, R * sizeof(int));
      alloc(&h->moe_row_gate, R * sizeof(float));
      alloc(&h->moe_pos, G * mb * sizeof(int));
      // hidden rows: row-major [R, h], or packed with every group on whole 256-row blocks
      // (prepared expert weights), at most G * pk_rows(max_batch) rows
      alloc(&h->moe_hidden, size_t(G) * size_t(pk_rows(int64_t(mb))) * size_t(cfg->moe_hidden) * 2);
      alloc(&h->moe_out, R * size_t(cfg->D) * 2);
    }
  }
  if (!ok) {
    rmx_destroy(h);
    return fail(nullptr, RMX_ERR_OUT_OF_MEMORY, "workspace allocation failed after %zu bytes", total);
  }
  *out_handle = h;
  return RMX_OK;
}

rmx_status rmx_destroy(rmx_handle* h) {
  if (!h) return RMX_OK;
  if (!h->allocs.empty() || !h->pending.empty() || !h->free_events.empty()) {
    (void)hipDeviceSynchronize();
  }
  for (void* q : h->allocs) (void)hipFree(q);
  for (auto& p : h->pending) {
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  for (auto e : h->free_events) (void)hipEventDestroy(e);
  delete h;
  return RMX_OK;
}

// Which prepared-operand paths a handle's configuration can run.
static void set_capabilities(rmx_handle* h) {
  const rmx_config* cfg = &h->cfg;
  h->pk_capable = cfg->moe_experts == 0 && cfg->dtype == RMX_BF16 && cfg->D % 32 == 0 &&
                  (int64_t(cfg->k) * cfg->D) % 32 == 0;
  h->mx_capable = h->pk_capable && cfg->D % 64 == 0 && (int64_t(cfg->k) * cfg->D) % 64 == 0;
  h->moe_pk_capable = cfg->moe_experts > 0 && cfg->dtype == RMX_BF16 && cfg->D % 384 == 0 &&
                      cfg->moe_hidden % 384 == 0 &&
                      gemm_moe_supported(cfg->moe_hidden, cfg->D, int64_t(cfg->T) * cfg->max_batch, true) &&
                      gemm_moe_supported(cfg->D, cfg->moe_hidden, cfg->max_batch, true);
}

// The forward pass; with `saved` (training) it also keeps S, U, H and the pre-LN2 rows of
// every block there instead of in the workspace.
static rmx_status forward_impl(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                               int32_t k, float* out, void* xl_out, float* gate_out, void* saved,
                               size_t saved_bytes, void* stream, const rmx_moe_lists* lists = nullptr) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  clear_error(h);
  const rmx_config& c = h->cfg;
  if (!w) return fail(h, RMX_ERR_INVALID_ARG, "weights is NULL");
  if (L != c.L) return fail(h, RMX_ERR_INVALID_ARG, "L=%d but the handle was created with L=%d", L, c.L);
  if (k != c.k) return fail(h, RMX_ERR_INVALID_ARG, "k=%d but the handle was created with k=%d", k, c.k);
  if (B < 0 || B > c.max_batch)
    return fail(h, RMX_ERR_INVALID_ARG, "B=%lld outside [0, max_batch=%lld]", (long long)B,
                (long long)c.max_batch);
  const bool moe = c.moe_experts > 0;
  const bool train = saved != nullptr;
  const bool attn = c.routing == RMX_ROUTING_ATTENTION;
  if (attn && (train || w->packed || w->packed_mxfp8))
    return fail(h, RMX_ERR_UNSUPPORTED, "attention routing runs the forward on W1 and W2 only");
  if (!attn && (w->Wq || w->Wk || w->Wv))
    return fail(h, RMX_ERR_INVALID_ARG, "Wq / Wk / Wv given to a Token Mixing handle");
  if (gate_out && !moe) return fail(h, RMX_ERR_INVALID_ARG, "gate_out must be NULL for a dense handle");
  if (lists && !moe) return fail(h, RMX_ERR_INVALID_ARG, "routing lists exist for Sparse-MoE handles only");
  if (train && moe) return fail(h, RMX_ERR_UNSUPPORTED, "training needs a dense handle");
  if (train && w->packed && !(w->W1 && w->W2))
    return fail(h, RMX_ERR_INVALID_ARG, "training needs W1 and W2 (the backward reads them) beside packed");
  if (train && saved_bytes < rmx_saved_bytes(h, B))
    return fail(h, RMX_ERR_INVALID_ARG, "saved buffer of %zu bytes, %zu needed", saved_bytes,
                rmx_saved_bytes(h, B));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  if (B == 0) return RMX_OK;

  const size_t esz = dtype_size(c.dtype);
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D, Ls = c.L;
  rmx_status st;
  if ((st = check_dev(h, X, size_t(B) * T * D * esz, dev, "X")) != RMX_OK) return st;
  if ((st = check_dev(h, out, size_t(B) * D * 4, dev, "out")) != RMX_OK) return st;
  if ((st = check_dev_opt(h, xl_out, size_t(B) * T * D * esz, dev, "xl_out")) != RMX_OK) return st;
  if (train && (st = check_dev(h, saved, rmx_saved_bytes(h, B), dev, "saved")) != RMX_OK) return st;
  const size_t E = size_t(c.moe_experts), hid = size_t(c.moe_hidden);
  if (moe) {
    if (w->packed_mxfp8) return fail(h, RMX_ERR_UNSUPPORTED, "MXFP8 weights are for dense handles");
    if ((st = check_dev(h, w->Wg, Ls * T * D * E * esz, dev, "Wg")) != RMX_OK) return st;
    if (w->packed) {
      if (!h->moe_pk_capable)
        return fail(h, RMX_ERR_UNSUPPORTED,
                    "prepared expert weights need a bf16 handle with D and moe_hidden multiples of 384");
      if ((st = check_dev(h, w->packed, rmx_packed_weights_bytes(h), dev, "packed")) != RMX_OK) return st;
    } else {
      if ((st = check_dev(h, w->We1, Ls * T * E * D * hid * esz, dev, "We1")) != RMX_OK) return st;
      if ((st = check_dev(h, w->We2, Ls * T * E * hid * D * esz, dev, "We2")) != RMX_OK) return st;
    }
    if ((st = check_dev_opt(h, w->be1, Ls * T * E * hid * esz, dev, "be1")) != RMX_OK) return st;
    if ((st = check_dev_opt(h, w->be2, Ls * T * E * D * esz, dev, "be2")) != RMX_OK) return st;
    if ((st = check_dev_opt(h, gate_out, Ls * size_t(B) * T * E * 4, dev, "gate_out")) != RMX_OK) return st;
    if (lists) {
      const size_t G = T * E;
      if ((st = check_dev_opt(h, lists->group_start, Ls * (G + 1) * 4, dev, "lists.group_start")) != RMX_OK ||
          (st = check_dev_opt(h, lists->rows, Ls * G * size_t(B) * 4, dev, "lists.rows")) != RMX_OK ||
          (st = check_dev_opt(h, lists->row_gate, Ls * G * size_t(B) * 4, dev, "lists.row_gate")) != RMX_OK ||
          (st = check_dev_opt(h, lists->pos, Ls * G * size_t(B) * 4, dev, "lists.pos")) != RMX_OK ||
          (st = check_dev_opt(h, lists->tile_start, Ls * (G + 1) * 4, dev, "lists.tile_start")) != RMX_OK)
        return st;
    }
  } else if (w->packed) {
    if (!h->pk_capable)
      return fail(h, RMX_ERR_UNSUPPORTED, "prepared weights need a dense bf16 handle with D and k*D multiples of 32");
    if ((st = check_dev(h, w->packed, rmx_packed_weights_bytes(h), dev, "packed")) != RMX_OK) return st;
    if (train) {
      if ((st = check_dev(h, w->W1, Ls * T * D * kD * esz, dev, "W1")) != RMX_OK) return st;
      if ((st = check_dev(h, w->W2, Ls * T * kD * D * esz, dev, "W2")) != RMX_OK) return st;
    }
  } else if (w->packed_mxfp8) {
    if (!h->mx_capable)
      return fail(h, RMX_ERR_UNSUPPORTED, "MXFP8 weights need a dense bf16 handle with D and k*D multiples of 64");
    if (train) return fail(h, RMX_ERR_INVALID_ARG, "training reads W1 and W2: packed_mxfp8 must be NULL");
    if ((st = check_dev(h, w->packed_mxfp8, rmx_packed_weights_mxfp8_bytes(h), dev, "packed_mxfp8")) != RMX_OK)
      return st;
  } else {
    if ((st = check_dev(h, w->W1, Ls * T * D * kD * esz, dev, "W1")) != RMX_OK) return st;
    if ((st = check_dev(h, w->W2, Ls * T * kD * D * esz, dev, "W2")) != RMX_OK) return st;
  }
  if (!moe) {
    if ((st = check_dev_opt(h, w->b1, Ls * T * kD * esz, dev, "b1")) != RMX_OK) return st;
    if ((st = check_dev_opt(h, w->b2, Ls * T * D * esz, dev, "b2")) != RMX_OK) return st;
    if (w->Wg || w->We1 || w->We2 || w->be1 || w->be2)
      return fail(h, RMX_ERR_INVALID_ARG, "MoE weights given to a dense handle");
  }
  if ((st = check_dev(h, w->ln1_g, Ls * D * esz, dev, "ln1_g")) != RMX_OK) return st;
  if ((st = check_dev(h, w->ln1_b, Ls * D * esz, dev, "ln1_b")) != RMX_OK) return st;
  if ((st = check_dev(h, w->ln2_g, Ls * D * esz, dev, "ln2_g")) != RMX_OK) return st;
  if ((st = check_dev(h, w->ln2_b, Ls * D * esz, dev, "ln2_b")) != RMX_OK) return st;
  if (attn) {
    if ((st = check_dev(h, w->Wq, Ls * D * D * esz, dev, "Wq")) != RMX_OK) return st;
    if ((st = check_dev(h, w->Wk, Ls * D * D * esz, dev, "Wk")) != RMX_OK) return st;
    if ((st = check_dev(h, w->Wv, Ls * D * D * esz, dev, "Wv")) != RMX_OK) return st;
  }
  // The outputs must not overlap the inputs: out and xl_out are written while X is read.
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
  };
  if (overlap(out, size_t(B) * D * 4, X, size_t(B) * T * D * esz) ||
      (xl_out && overlap(xl_out, size_t(B) * T * D * esz, X, size_t(B) * T * D * esz)) ||
      (xl_out && overlap(xl_out, size_t(B) * T * D * esz, out, size_t(B) * D * 4)))
    return fail(h, RMX_ERR_INVALID_ARG, "out / xl_out overlap X or each other");
  const SavedLayout lay = saved_layout(c, B);
  if (train) {
    const size_t sb = rmx_saved_bytes(h, B);
    if (overlap(saved, sb, X, size_t(B) * T * D * esz) || overlap(saved, sb, out, size_t(B) * D * 4) ||
        (xl_out && overlap(saved, sb, xl_out, size_t(B) * T * D * esz)))
      return fail(h, RMX_ERR_INVALID_ARG, "saved overlaps X, out or xl_out");
  }
  // block n's S, hidden and pre-LN2 rows: the saved activations (training) or the workspace
  auto blk = [&](int n, size_t off) { return static_cast<char*>(saved) + size_t(n) * lay.per_block + off; };
  auto S_of = [&](int n) -> void* { return train ? blk(n, lay.S) : h->S; };
  auto H_of = [&](int n) -> void* { return train ? blk(n, lay.H) : h->H; };
  auto Y_of = [&](int n) -> float* { return train ? reinterpret_cast<float*>(blk(n, lay.Y)) : h->Y; };
  // After a Sparse-MoE block the next row pass forms the pre-LN2 rows itself from that
  // block's S and gate-scaled expert rows (no Y in memory).
  auto moe_combine_rows = [&](RowsArgs& ra) {
    if (!moe) return;
    ra.in = h->S;
    ra.moe_ye = h->moe_out;
    ra.moe_pos = h->moe_pos;
    ra.moe_E = c.moe_experts;
  };

  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* bytes = nullptr;
  auto at = [&](const void* base, size_t off_elems) -> const void* {
    if (!base) return nullptr;
    bytes = static_cast<const char*>(base);
    return bytes + off_elems * esz;
  };
  hipError_t e = hipSuccess;
  const int Bi = int(B);
  const bool pk = !moe && !train && w->packed != nullptr;
  // training on prepared weights: the products read W from the prepared copy and S, H
  // row-major (the saved activations), where their shapes allow 384-wide tiles; the same bits
  const bool pk_train1 = train && !moe && w->packed != nullptr && gemm_packed_w_supported(B, int64_t(kD), int64_t(D));
  const bool pk_train2 = train && !moe && w->packed != nullptr && gemm_packed_w_supported(B, int64_t(D), int64_t(kD));
  const bool moe_pk = moe && w->packed != nullptr;
  // prepared expert weights of block n: the T*E groups' We1^T, then their We2^T (elements)
  const size_t pk_we1 = T * E * size_t(pk_rows(int64_t(hid))) * D, pk_we2 = T * E * size_t(pk_rows(int64_t(D))) * hid;
  const bool mx = !moe && !pk && w->packed_mxfp8 != nullptr;
  // prepared weights of block n: W1^T then W2^T, packed (elements)
  const size_t pk_w1 = T * size_t(pk_rows(int64_t(kD))) * D, pk_w2 = T * size_t(pk_rows(int64_t(D))) * kD;
  // MXFP8 weights of block n (bytes): W1^T codes, their scales, W2^T codes, their scales;
  // S and H in MXFP8: codes, then scales
  const size_t mx_w1 = pk_w1, mx_w2 = pk_w2, mx_blk = (mx_w1 + mx_w2) / 32 * 33;
  const size_t pkB = size_t(pk_rows(B));
  char* S8 = static_cast<char*>(h->S8);
  char* H8 = static_cast<char*>(h->H);
  for (int n = 0; n < c.L && e == hipSuccess; ++n) {
    if (attn) {
      // block input: X, or LN2 of the previous block written out by the pooling row launch
      const void* Xn = X;
      if (n > 0) {
        RowsArgs ra{};
        ra.in = Y_of(n - 1);
        ra.ln2_g = at(w->ln2_g, size_t(n - 1) * D);
        ra.ln2_b = at(w->ln2_b, size_t(n - 1) * D);
        ra.pool = h->a_pool;
        ra.xl = h->aX;
        ra.B = Bi;
        ra.T = c.T;
        ra.D = c.D;
        ra.eps = c.ln_eps;
        if ((e = run_rows(h, s, ROWS_FINAL, ra)) != hipSuccess) break;
        Xn = h->aX;
      }
      // Q, K, V over the B*T rows, one product each (no bias)
      void* qkv[3] = {h->aQ, h->aK, h->aV};
      const void* wqkv[3] = {w->Wq, w->Wk, w->Wv};
      for (int m = 0; m < 3 && e == hipSuccess; ++m) {
        GemmArgs pa{};
        pa.A = Xn;
        pa.W = at(wqkv[m], size_t(n) * D * D);
        pa.C = qkv[m];
        pa.G = 1;
        pa.M = Bi * c.T;
        pa.N = c.D;
        pa.K = c.D;
        e = run_gemm(h, s, EPI_BIAS, pa, RMX_KERNEL_ATTN_QKV);
      }
      if (e != hipSuccess) break;
      AttnArgs aa{};
      aa.Q = h->aQ;
      aa.K = h->aK;
      aa.V = h->aV;
      aa.X = Xn;
      aa.ln1_g = at(w->ln1_g, size_t(n) * D);
      aa.ln1_b = at(w->ln1_b, size_t(n) * D);
      aa.S = h->S;
      aa.B = Bi;
      aa.T = c.T;
      aa.D = c.D;
      aa.eps = c.ln_eps;
      if ((e = run_attn(h, s, aa)) != hipSuccess) break;
    } else {
      RowsArgs ra{};
      ra.in = n == 0 ? X : static_cast<const void*>(Y_of(n - 1));
      if (n > 0) moe_combine_rows(ra);
      ra.ln2_g = n == 0 ? nullptr : at(w->ln2_g, size_t(n - 1) * D);
      ra.ln2_b = n == 0 ? nullptr : at(w->ln2_b, size_t(n - 1) * D);
      ra.ln1_g = at(w->ln1_g, size_t(n) * D);
      ra.ln1_b = at(w->ln1_b, size_t(n) * D);
      ra.S = S_of(n);
      ra.B = Bi;
      ra.T = c.T;
      ra.D = c.D;
      ra.eps = c.ln_eps;
      ra.s_packed = (pk || mx) ? 1 : 0;
      if (mx) {
        ra.s8 = S8;
        ra.s8_scale = S8 + T * pkB * D;
      }
      e = run_rows(h, s, n == 0 ? ROWS_FIRST : ROWS_MID, ra);
      if (e != hipSuccess) break;
    }

    if (moe) {
      // Sparse-MoE PFFN: route, expert FFN1 over gathered rows, gate-scaled FFN2, combine.
      MoeArgs ma{};
      ma.S = h->S;
      ma.Wg = at(w->Wg, size_t(n) * T * D * E);
      ma.g = h->moe_g;
      ma.gate_out = gate_out ? gate_out + size_t(n) * size_t(B) * T * E : nullptr;
      ma.cnt = h->moe_cnt;
      ma.chunk_off = h->moe_chunk_off;
      ma.group_rows = h->moe_group_rows;
      ma.group_start = h->moe_group_start;
      ma.tile_start = h->moe_tile_start;
      ma.src_row = h->moe_src_row;
      ma.row_gate = h->moe_row_gate;
      ma.pos = h->moe_pos;
      ma.B = Bi;
      ma.T = c.T;
      ma.D = c.D;
      ma.E = c.moe_experts;
      ma.nchunk = (Bi + 63) / 64;
      if ((e = run_moe_route(h, s, ma)) != hipSuccess) break;
      if (lists) {
        // diagnostic copies of this block's routing lists (device to device, on the stream)
        const size_t G = T * E, GB = G * size_t(B);
        auto cp = [&](void* dst, const void* src, size_t bytes) {
          if (dst && e == hipSuccess) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
        };
        cp(lists->group_start ? lists->group_start + size_t(n) * (G + 1) : nullptr, h->moe_group_start,
           (G + 1) * 4);
        cp(lists->rows ? lists->rows + size_t(n) * GB : nullptr, h->moe_src_row, GB * 4);
        cp(lists->row_gate ? lists->row_gate + size_t(n) * GB : nullptr, h->moe_row_gate, GB * 4);
        cp(lists->pos ? lists->pos + size_t(n) * GB : nullptr, h->moe_pos, GB * 4);
        cp(lists->tile_start ? lists->tile_start + size_t(n) * (G + 1) : nullptr, h->moe_tile_start, (G + 1) * 4);
        if (e != hipSuccess) break;
      }
      const uint16_t* pkw = moe_pk ? static_cast<const uint16_t*>(w->packed) + size_t(n) * (pk_we1 + pk_we2) : nullptr;
      GemmArgs m1{};
      m1.A = h->S;
      m1.W = moe_pk ? static_cast<const void*>(pkw) : at(w->We1, size_t(n) * T * E * D * hid);
      m1.packed = moe_pk ? 1 : 0;
      m1.bias = at(w->be1, size_t(n) * T * E * hid);
      m1.C = h->moe_hidden;
      m1.G = int(T * E);
      m1.N = int(hid);
      m1.K = c.D;
      m1.group_start = h->moe_group_start;
      m1.tile_start = h->moe_tile_start;
      m1.src_row = h->moe_src_row;
      m1.a_rows = int(T) * Bi;
      if ((e = run_moe_gemm(h, s, EPI_MOE1, m1)) != hipSuccess) break;
      GemmArgs m2{};
      m2.A = h->moe_hidden;
      m2.W = moe_pk ? static_cast<const void*>(pkw + pk_we1) : at(w->We2, size_t(n) * T * E * hid * D);
      m2.packed = moe_pk ? 1 : 0;
      m2.bias = at(w->be2, size_t(n) * T * E * D);
      m2.C = h->moe_out;
      m2.G = int(T * E);
      m2.N = c.D;
      m2.K = int(hid);
      m2.group_start = h->moe_group_start;
      m2.tile_start = h->moe_tile_start;
      m2.row_gate = h->moe_row_gate;
      // the combine S + sum of the gate-scaled expert rows runs inside the next row pass
      e = run_moe_gemm(h, s, EPI_MOE2, m2);
      continue;
    }

    if (mx) {
      const char* wb = static_cast<const char*>(w->packed_mxfp8) + size_t(n) * mx_blk;
      GemmArgs m1{};
      m1.A = S8;
      m1.A_scale = S8 + T * pkB * D;
      m1.W = wb;
      m1.W_scale = wb + mx_w1;
      m1.bias = at(w->b1, size_t(n) * T * kD);
      m1.C = H8;
      m1.C_scale = H8 + T * pkB * kD;
      m1.G = c.T;
      m1.M = Bi;
      m1.N = int(kD);
      m1.K = c.D;
      if ((e = run_gemm_mx(h, s, EPI_GELU_MX, m1)) != hipSuccess) break;
      GemmArgs m2{};
      m2.A = H8;
      m2.A_scale = H8 + T * pkB * kD;
      m2.W = wb + mx_w1 / 32 * 33;
      m2.W_scale = wb + mx_w1 / 32 * 33 + mx_w2;
      m2.bias = at(w->b2, size_t(n) * T * D);
      m2.R = h->S;
      m2.C = h->Y;
      m2.G = c.T;
      m2.M = Bi;
      m2.N = c.D;
      m2.K = int(kD);
      e = run_gemm_mx(h, s, EPI_RESID, m2);
      continue;
    }

    GemmArgs g1{};
    g1.A = S_of(n);
    g1.W = (pk || pk_train1) ? at(w->packed, size_t(n) * (pk_w1 + pk_w2)) : at(w->W1, size_t(n) * T * D * kD);
    g1.packed = pk ? 1 : (pk_train1 ? GEMM_PACKED_W : 0);
    g1.bias = at(w->b1, size_t(n) * T * kD);
    g1.C = H_of(n);
    g1.U = train ? blk(n, lay.U) : nullptr;
    g1.G = c.T;
    g1.M = Bi;
    g1.N = int(kD);
    g1.K = c.D;
    e = run_gemm(h, s, train ? EPI_GELU_SAVE : EPI_GELU, g1);
    if (e != hipSuccess) break;

    GemmArgs g2{};
    g2.A = H_of(n);
    g2.W = (pk || pk_train2) ? at(w->packed, size_t(n) * (pk_w1 + pk_w2) + pk_w1) : at(w->W2, size_t(n) * T * kD * D);
    g2.packed = pk ? 1 : (pk_train2 ? GEMM_PACKED_W : 0);
    g2.bias = at(w->b2, size_t(n) * T * D);
    g2.R = S_of(n);
    g2.C = Y_of(n);
    g2.G = c.T;
    g2.M = Bi;
    g2.N = c.D;
    g2.K = int(kD);
    e = run_gemm(h, s, EPI_RESID, g2);
  }
  if (e == hipSuccess) {
    RowsArgs ra{};
    ra.in = Y_of(c.L - 1);
    moe_combine_rows(ra);
    ra.ln2_g = at(w->ln2_g, size_t(c.L - 1) * D);
    ra.ln2_b = at(w->ln2_b, size_t(c.L - 1) * D);
    ra.pool = out;
    ra.xl = xl_out;
    ra.B = Bi;
    ra.T = c.T;
    ra.D = c.D;
    ra.eps = c.ln_eps;
    e = run_rows(h, s, ROWS_FINAL, ra);
  }
  if (e != hipSuccess) return fail(h, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMX_OK;
}

rmx_status rmx_block_forward_ex(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w,
                                int32_t L, int32_t k, float* out, void* xl_out, float* gate_out,
                                void* stream) {
  return forward_impl(h, X, B, w, L, k, out, xl_out, gate_out, nullptr, 0, stream);
}

rmx_status rmx_block_forward_moe_lists(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w,
                                       int32_t L, int32_t k, float* out, void* xl_out, float* gate_out,
                                       const rmx_moe_lists* lists, void* stream) {
  if (!lists) {
    if (h) clear_error(h);
    return fail(h, RMX_ERR_INVALID_ARG, "lists is NULL");
  }
  return forward_impl(h, X, B, w, L, k, out, xl_out, gate_out, nullptr, 0, stream, lists);
}

size_t rmx_saved_bytes(const rmx_handle* h, int64_t B) {
  if (!h || B < 0 || h->cfg.moe_experts > 0) return 0;
  return size_t(h->cfg.L) * saved_layout(h->cfg, B).per_block;
}

rmx_status rmx_block_forward_train(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                                   int32_t k, float* out, void* saved, size_t saved_bytes, void* stream) {
  if (!saved) {
    if (h) clear_error(h);
    return fail(h, RMX_ERR_INVALID_ARG, "saved is NULL");
  }
  return forward_impl(h, X, B, w, L, k, out, nullptr, nullptr, saved, saved_bytes, stream);
}

// The backward workspace, for max_batch samples; allocated once per handle.
static rmx_status ensure_bwd_workspace(rmx_handle* h) {
  if (h->bwd_ready) return RMX_OK;
  const rmx_config& c = h->cfg;
  const size_t esz = dtype_size(c.dtype), rows = size_t(c.T) * size_t(c.max_batch);
  const size_t D = c.D, kD = size_t(c.k) * c.D;
  std::vector<void*> got;
  bool ok = true;
  auto alloc = [&](auto** ptr, size_t bytes) {
    if (!ok) return;
    void* q = nullptr;
    if (hipMalloc(&q, bytes ? bytes : 16) != hipSuccess) {
      (void)hipGetLastError();
      ok = false;
      return;
    }
    got.push_back(q);
    *ptr = static_cast<std::remove_pointer_t<std::remove_reference_t<decltype(*ptr)>>*>(q);
  };
  alloc(&h->bw_gY32, rows * D * 4);
  alloc(&h->bw_gY, rows * D * esz);
  alloc(&h->bw_gU, rows * kD * esz);
  alloc(&h->bw_gS, rows * D * 4);
  alloc(&h->bw_gR, rows * D * 4);
  alloc(&h->bw_part1, 2 * size_t(c.max_batch) * D * 4);
  alloc(&h->bw_part2, 2 * size_t(c.max_batch) * D * 4);
  alloc(&h->bw_sum, colsum_scratch_floats(c.T, c.max_batch, int64_t(kD > D ? kD : D)) * 4);
  alloc(&h->bw_cpart, size_t(c.T) * colsum_rows(int(c.max_batch)) * (kD > D ? kD : D) * 4);
  if (!ok) {
    for (void* q : got) (void)hipFree(q);
    h->bw_gY32 = h->bw_gS = h->bw_gR = h->bw_part1 = h->bw_part2 = h->bw_sum = h->bw_cpart = nullptr;
    h->bw_gY = h->bw_gU = nullptr;
    return fail(h, RMX_ERR_OUT_OF_MEMORY, "backward workspace allocation failed");
  }
  h->allocs.insert(h->allocs.end(), got.begin(), got.end());
  h->bwd_ready = true;
  return RMX_OK;
}

rmx_status rmx_block_backward(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                              int32_t k, const void* saved, size_t saved_bytes, const float* g_out, float* dX,
                              const rmx_grads* grads, void* stream) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  clear_error(h);
  const rmx_config& c = h->cfg;
  if (!w) return fail(h, RMX_ERR_INVALID_ARG, "weights is NULL");
  if (!grads) return fail(h, RMX_ERR_INVALID_ARG, "grads is NULL");
  if (L != c.L) return fail(h, RMX_ERR_INVALID_ARG, "L=%d but the handle was created with L=%d", L, c.L);
  if (k != c.k) return fail(h, RMX_ERR_INVALID_ARG, "k=%d but the handle was created with k=%d", k, c.k);
  if (B < 0 || B > c.max_batch)
    return fail(h, RMX_ERR_INVALID_ARG, "B=%lld outside [0, max_batch=%lld]", (long long)B,
                (long long)c.max_batch);
  if (c.moe_experts > 0) return fail(h, RMX_ERR_UNSUPPORTED, "the backward needs a dense handle");
  // the backward reads W1 and W2 (w->packed, if set, is the forward's prepared copy: unused)
  if (!rows_bwd_supported(c.dtype, c.T, c.D))
    return fail(h, RMX_ERR_UNSUPPORTED, "the backward row kernel takes D <= %d (D %% 8 == 0, (D/T) %% 8 == 0) or "
                "D <= %d, and T*D*sizeof(dtype) within its LDS", ROWS_BWD_MAX_D, ROWS_BWD_MAX_D_SCALAR);
  const size_t need = rmx_saved_bytes(h, B);
  if (saved_bytes < need) return fail(h, RMX_ERR_INVALID_ARG, "saved buffer of %zu bytes, %zu needed", saved_bytes, need);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  if (B == 0) return RMX_OK;

  const size_t esz = dtype_size(c.dtype);
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D, Ls = c.L, Bs = size_t(B);
  struct Span {
    const void* p;
    size_t bytes;
    const char* name;
  };
  const Span ins[] = {{X, Bs * T * D * esz, "X"},          {saved, need, "saved"},
                      {g_out, Bs * D * 4, "g_out"},        {w->W1, Ls * T * D * kD * esz, "W1"},
                      {w->W2, Ls * T * kD * D * esz, "W2"}, {w->ln1_g, Ls * D * esz, "ln1_g"},
                      {w->ln2_g, Ls * D * esz, "ln2_g"},    {w->ln2_b, Ls * D * esz, "ln2_b"}};
  const Span outs[] = {{dX, Bs * T * D * 4, "dX"},
                       {grads->dW1, Ls * T * D * kD * 4, "dW1"},
                       {grads->db1, Ls * T * kD * 4, "db1"},
                       {grads->dW2, Ls * T * kD * D * 4, "dW2"},
                       {grads->db2, Ls * T * D * 4, "db2"},
                       {grads->dln1_g, Ls * D * 4, "dln1_g"},
                       {grads->dln1_b, Ls * D * 4, "dln1_b"},
                       {grads->dln2_g, Ls * D * 4, "dln2_g"},
                       {grads->dln2_b, Ls * D * 4, "dln2_b"}};
  rmx_status st;
  for (const Span& x : ins)
    if ((st = check_dev(h, x.p, x.bytes, dev, x.name)) != RMX_OK) return st;
  for (const Span& x : outs)
    if ((st = check_dev(h, x.p, x.bytes, dev, x.name)) != RMX_OK) return st;
  auto overlap = [](const Span& a, const Span& b) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + b.bytes && y < x + a.bytes;
  };
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Span& x : ins)
      if (overlap(outs[i], x)) return fail(h, RMX_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, x.name);
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(h, RMX_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  if ((st = ensure_bwd_workspace(h)) != RMX_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const SavedLayout lay = saved_layout(c, B);
  auto blk = [&](int n, size_t off) {
    return const_cast<char*>(static_cast<const char*>(saved)) + size_t(n) * lay.per_block + off;
  };
  auto at = [&](const void* base, size_t off_elems) -> const void* {
    return static_cast<const char*>(base) + off_elems * esz;
  };
  const int Bi = int(B), Ti = c.T, Di = c.D, kDi = int(kD);
  hipError_t e = hipSuccess;
  auto ln_sums = [&](const float* part, float* dg, float* db) {
    if (e == hipSuccess) e = run_colsum(h, s, DT_FP32, part, dg, 1, Bi, Di);
    if (e == hipSuccess) e = run_colsum(h, s, DT_FP32, part + Bs * D, db, 1, Bi, Di);
  };
  for (int n = c.L - 1; n >= 0 && e == hipSuccess; --n) {
    const size_t nn = size_t(n);
    void* S_n = blk(n, lay.S);
    void* G_n = blk(n, lay.U);  // GELU' at the pre-activations
    void* H_n = blk(n, lay.H);
    if (n == c.L - 1) {
      // gradient of the last block's pre-LN2 rows from the pooled output's
      RowsBwdArgs ra{};
      ra.Y = reinterpret_cast<const float*>(blk(n, lay.Y));
      ra.ln2_g = at(w->ln2_g, nn * D);
      ra.g_out = g_out;
      ra.gY32 = h->bw_gY32;
      ra.gY = h->bw_gY;
      ra.part_ln2 = h->bw_part2;
      ra.B = Bi;
      ra.T = Ti;
      ra.D = Di;
      ra.eps = c.ln_eps;
      e = run_rows_bwd(h, s, BWD_TOP, ra);
      ln_sums(h->bw_part2, grads->dln2_g + nn * D, grads->dln2_b + nn * D);
      if (e != hipSuccess) break;
    }
    // gU = (gY W2^T) * GELU'(U); db1 = sum over samples of gU (column sums of the matrix-core
    // epilogue, else a pass over gU)
    GemmArgs du{};
    du.A = h->bw_gY;
    du.W = at(w->W2, nn * T * kD * D);
    du.bt = 1;
    du.R = G_n;
    du.C = h->bw_gU;
    du.G = Ti;
    du.M = Bi;
    du.N = kDi;
    du.K = Di;
    const bool du_sums = gemm_writes_colsum(c.dtype, EPI_GELU_BWD, du);
    du.colsum = du_sums ? h->bw_cpart : nullptr;
    if ((e = run_gemm(h, s, EPI_GELU_BWD, du, RMX_KERNEL_BWD_DU)) != hipSuccess) break;
    e = du_sums ? run_colsum(h, s, DT_FP32, h->bw_cpart, grads->db1 + nn * T * kD, Ti, colsum_rows(Bi), kDi)
                : run_colsum(h, s, c.dtype, h->bw_gU, grads->db1 + nn * T * kD, Ti, Bi, kDi);
    if (e != hipSuccess) break;
    // dW2 = H^T gY
    GemmArgs dw2{};
    dw2.A = H_n;
    dw2.at = 1;
    dw2.W = h->bw_gY;
    dw2.C = grads->dW2 + nn * T * kD * D;
    dw2.G = Ti;
    dw2.M = kDi;
    dw2.N = Di;
    dw2.K = Bi;
    if ((e = run_gemm(h, s, EPI_STORE32, dw2, RMX_KERNEL_BWD_DW2)) != hipSuccess) break;
    // dW1 = S^T gU
    GemmArgs dw1{};
    dw1.A = S_n;
    dw1.at = 1;
    dw1.W = h->bw_gU;
    dw1.C = grads->dW1 + nn * T * D * kD;
    dw1.G = Ti;
    dw1.M = Di;
    dw1.N = kDi;
    dw1.K = Bi;
    if ((e = run_gemm(h, s, EPI_STORE32, dw1, RMX_KERNEL_BWD_DW1)) != hipSuccess) break;
    // gS = gU W1^T + gY (the second residual)
    GemmArgs ds{};
    ds.A = h->bw_gU;
    ds.W = at(w->W1, nn * T * D * kD);
    ds.bt = 1;
    ds.R = h->bw_gY32;
    ds.C = h->bw_gS;
    ds.G = Ti;
    ds.M = Bi;
    ds.N = Di;
    ds.K = kDi;
    // db2 = sum over samples of the pre-LN2 row gradients (the residual this product reads)
    const bool ds_sums = gemm_writes_colsum(c.dtype, EPI_RESID32, ds);
    ds.colsum = ds_sums ? h->bw_cpart : nullptr;
    if ((e = run_gemm(h, s, EPI_RESID32, ds, RMX_KERNEL_BWD_DS)) != hipSuccess) break;
    e = ds_sums ? run_colsum(h, s, DT_FP32, h->bw_cpart, grads->db2 + nn * T * D, Ti, colsum_rows(Bi), Di)
                : run_colsum(h, s, DT_FP32, h->bw_gY32, grads->db2 + nn * T * D, Ti, Bi, Di);
    if (e != hipSuccess) break;
    // LN1 backward, mixing transpose and first residual; then LN2 backward of block n - 1
    RowsBwdArgs ra{};
    ra.ln1_g = at(w->ln1_g, nn * D);
    ra.gS = h->bw_gS;
    ra.gR = h->bw_gR;
    ra.part_ln1 = h->bw_part1;
    ra.B = Bi;
    ra.T = Ti;
    ra.D = Di;
    ra.eps = c.ln_eps;
    if (n > 0) {
      ra.Y = reinterpret_cast<const float*>(blk(n - 1, lay.Y));
      ra.ln2_g = at(w->ln2_g, (nn - 1) * D);
      ra.ln2_b = at(w->ln2_b, (nn - 1) * D);
      ra.gY32 = h->bw_gY32;
      ra.gY = h->bw_gY;
      ra.part_ln2 = h->bw_part2;
      e = run_rows_bwd(h, s, BWD_MID, ra);
      ln_sums(h->bw_part1, grads->dln1_g + nn * D, grads->dln1_b + nn * D);
      ln_sums(h->bw_part2, grads->dln2_g + (nn - 1) * D, grads->dln2_b + (nn - 1) * D);
    } else {
      ra.X0 = X;
      ra.dX = dX;
      e = run_rows_bwd(h, s, BWD_BOTTOM, ra);
      ln_sums(h->bw_part1, grads->dln1_g, grads->dln1_b);
    }
  }
  if (e != hipSuccess) return fail(h, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMX_OK;
}

size_t rmx_packed_weights_bytes(const rmx_handle* h) {
  if (!h) return 0;
  const rmx_config& c = h->cfg;
  if (h->moe_pk_capable) {
    const size_t G = size_t(c.T) * size_t(c.moe_experts), D = c.D, hid = c.moe_hidden;
    return size_t(c.L) * G * (size_t(pk_rows(int64_t(hid))) * D + size_t(pk_rows(int64_t(D))) * hid) * 2;
  }
  if (!h->pk_capable) return 0;
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D;
  const size_t per_layer = T * size_t(pk_rows(int64_t(kD))) * D + T * size_t(pk_rows(int64_t(D))) * kD;
  return size_t(c.L) * per_layer * 2;
}

rmx_status rmx_pack_weights(rmx_handle* h, const rmx_weights* w, int32_t L, void* packed, size_t bytes,
                            void* stream) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  clear_error(h);
  const rmx_config& c = h->cfg;
  if (!w) return fail(h, RMX_ERR_INVALID_ARG, "weights is NULL");
  if (L != c.L) return fail(h, RMX_ERR_INVALID_ARG, "L=%d but the handle was created with L=%d", L, c.L);
  if (c.moe_experts > 0 && !h->moe_pk_capable)
    return fail(h, RMX_ERR_UNSUPPORTED,
                "prepared expert weights need a bf16 handle with D and moe_hidden multiples of 384");
  if (c.moe_experts == 0 && !h->pk_capable)
    return fail(h, RMX_ERR_UNSUPPORTED, "prepared weights need a dense bf16 handle with D and k*D multiples of 32");
  const size_t need = rmx_packed_weights_bytes(h);
  if (bytes < need) return fail(h, RMX_ERR_INVALID_ARG, "packed buffer of %zu bytes, %zu needed", bytes, need);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D, Ls = c.L;
  rmx_status st;
  const uintptr_t pb = reinterpret_cast<uintptr_t>(packed);
  if (c.moe_experts > 0) {
    // each expert's We1 [D, hid] and We2 [hid, D], groups t * E + e, as the dense W1 / W2
    const size_t G = T * size_t(c.moe_experts), hid = c.moe_hidden;
    const size_t src = Ls * G * D * hid * 2;
    if ((st = check_dev(h, w->We1, src, dev, "We1")) != RMX_OK) return st;
    if ((st = check_dev(h, w->We2, src, dev, "We2")) != RMX_OK) return st;
    if ((st = check_dev(h, packed, need, dev, "packed")) != RMX_OK) return st;
    for (const void* p : {w->We1, w->We2}) {
      const uintptr_t sb = reinterpret_cast<uintptr_t>(p);
      if (pb < sb + src && sb < pb + need) return fail(h, RMX_ERR_INVALID_ARG, "packed overlaps We1 or We2");
    }
    const size_t pk1 = G * size_t(pk_rows(int64_t(hid))) * D, pk2 = G * size_t(pk_rows(int64_t(D))) * hid;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t n = 0; n < Ls; ++n) {
      uint16_t* dst = static_cast<uint16_t*>(packed) + n * (pk1 + pk2);
      hipError_t e = launch_pack_weights(static_cast<const uint16_t*>(w->We1) + n * G * D * hid, dst, int(G), c.D,
                                         int(hid), s);
      if (e == hipSuccess)
        e = launch_pack_weights(static_cast<const uint16_t*>(w->We2) + n * G * hid * D, dst + pk1, int(G), int(hid),
                                c.D, s);
      if (e != hipSuccess) return fail(h, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return RMX_OK;
  }
  if ((st = check_dev(h, w->W1, Ls * T * D * kD * 2, dev, "W1")) != RMX_OK) return st;
  if ((st = check_dev(h, w->W2, Ls * T * kD * D * 2, dev, "W2")) != RMX_OK) return st;
  if ((st = check_dev(h, packed, need, dev, "packed")) != RMX_OK) return st;
  for (const void* src : {w->W1, w->W2}) {
    const uintptr_t sb = reinterpret_cast<uintptr_t>(src);
    if (pb < sb + Ls * T * D * kD * 2 && sb < pb + need)
      return fail(h, RMX_ERR_INVALID_ARG, "packed overlaps W1 or W2");
  }
  const size_t pk_w1 = T * size_t(pk_rows(int64_t(kD))) * D, pk_w2 = T * size_t(pk_rows(int64_t(D))) * kD;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t n = 0; n < Ls; ++n) {
    uint16_t* dst = static_cast<uint16_t*>(packed) + n * (pk_w1 + pk_w2);
    hipError_t e = launch_pack_weights(static_cast<const uint16_t*>(w->W1) + n * T * D * kD, dst, c.T, c.D, int(kD), s);
    if (e == hipSuccess)
      e = launch_pack_weights(static_cast<const uint16_t*>(w->W2) + n * T * kD * D, dst + pk_w1, c.T, int(kD), c.D, s);
    if (e != hipSuccess) return fail(h, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return RMX_OK;
}

size_t rmx_packed_weights_mxfp8_bytes(const rmx_handle* h) {
  if (!h || !h->mx_capable) return 0;
  const rmx_config& c = h->cfg;
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D;
  const size_t codes = T * size_t(pk_rows(int64_t(kD))) * D + T * size_t(pk_rows(int64_t(D))) * kD;
  return size_t(c.L) * (codes / 32 * 33);
}

rmx_status rmx_pack_weights_mxfp8(rmx_handle* h, const rmx_weights* w, int32_t L, void* packed, size_t bytes,
                                  void* stream) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  clear_error(h);
  const rmx_config& c = h->cfg;
  if (!w) return fail(h, RMX_ERR_INVALID_ARG, "weights is NULL");
  if (L != c.L) return fail(h, RMX_ERR_INVALID_ARG, "L=%d but the handle was created with L=%d", L, c.L);
  if (!h->mx_capable)
    return fail(h, RMX_ERR_UNSUPPORTED, "MXFP8 weights need a dense bf16 handle with D and k*D multiples of 64");
  const size_t need = rmx_packed_weights_mxfp8_bytes(h);
  if (bytes < need) return fail(h, RMX_ERR_INVALID_ARG, "packed buffer of %zu bytes, %zu needed", bytes, need);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return fail(h, RMX_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  }
  const size_t T = c.T, D = c.D, kD = size_t(c.k) * c.D, Ls = c.L;
  rmx_status st;
  if ((st = check_dev(h, w->W1, Ls * T * D * kD * 2, dev, "W1")) != RMX_OK) return st;
  if ((st = check_dev(h, w->W2, Ls * T * kD * D * 2, dev, "W2")) != RMX_OK) return st;
  if ((st = check_dev(h, packed, need, dev, "packed")) != RMX_OK) return st;
  const uintptr_t pb = reinterpret_cast<uintptr_t>(packed);
  for (const void* src : {w->W1, w->W2}) {
    const uintptr_t sb = reinterpret_cast<uintptr_t>(src);
    if (pb < sb + Ls * T * D * kD * 2 && sb < pb + need)
      return fail(h, RMX_ERR_INVALID_ARG, "packed overlaps W1 or W2");
  }
  // per block: W1^T codes [T][pk_rows(kD) x D], their scales, W2^T codes [T][pk_rows(D) x kD],
  // their scales
  const size_t c1 = T * size_t(pk_rows(int64_t(kD))) * D, c2 = T * size_t(pk_rows(int64_t(D))) * kD;
  const size_t blk = (c1 + c2) / 32 * 33;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t n = 0; n < Ls; ++n) {
    char* dst = static_cast<char*>(packed) + n * blk;
    hipError_t e = launch_pack_weights_mx(static_cast<const uint16_t*>(w->W1) + n * T * D * kD, dst, dst + c1, c.T,
                                          c.D, int(kD), s);
    if (e == hipSuccess)
      e = launch_pack_weights_mx(static_cast<const uint16_t*>(w->W2) + n * T * kD * D, dst + c1 / 32 * 33,
                                 dst + c1 / 32 * 33 + c2, c.T, int(kD), c.D, s);
    if (e != hipSuccess) return fail(h, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return RMX_OK;
}

rmx_status rmx_block_forward(rmx_handle* h, const void* X, int64_t B, const rmx_weights* w, int32_t L,
                             int32_t k, float* out, void* stream) {
  return rmx_block_forward_ex(h, X, B, w, L, k, out, nullptr, nullptr, stream);
}

rmx_status rmx_token_mix(const void* X, void* Y, int64_t B, int32_t T, int32_t D, int32_t dtype,
                         void* stream) {
  clear_error(nullptr);
  if (T < 1 || D < 1 || B < 0) return fail(nullptr, RMX_ERR_INVALID_ARG, "T, D must be >= 1 and B >= 0");
  if (D % T) return fail(nullptr, RMX_ERR_INVALID_ARG, "D=%d is not divisible by H=T=%d", D, T);
  if (dtype != RMX_FP32 && dtype != RMX_BF16) return fail(nullptr, RMX_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (B == 0) return RMX_OK;
  int dev = -1;
  rmx_status st = check_device_arch(nullptr, &dev);
  if (st != RMX_OK) return st;
  const size_t bytes = size_t(B) * T * D * dtype_size(dtype);
  if ((st = check_dev(nullptr, X, bytes, dev, "X")) != RMX_OK) return st;
  if ((st = check_dev(nullptr, Y, bytes, dev, "Y")) != RMX_OK) return st;
  const uintptr_t x = reinterpret_cast<uintptr_t>(X), y = reinterpret_cast<uintptr_t>(Y);
  if (x < y + bytes && y < x + bytes) return fail(nullptr, RMX_ERR_INVALID_ARG, "X and Y overlap");
  hipError_t e = launch_token_mix(dtype, X, Y, B, T, D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMX_OK;
}

rmx_status rmx_tokenize(const void* E, const void* Wp, const void* bp, void* X, int64_t B, int32_t T,
                        int32_t d, int32_t D, int32_t dtype, void* stream) {
  clear_error(nullptr);
  if (T < 1 || d < 1 || D < 1 || B < 0) return fail(nullptr, RMX_ERR_INVALID_ARG, "T, d, D must be >= 1 and B >= 0");
  if (dtype != RMX_FP32 && dtype != RMX_BF16) return fail(nullptr, RMX_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (B > INT32_MAX) return fail(nullptr, RMX_ERR_UNSUPPORTED, "B must be < 2^31");
  if (B == 0) return RMX_OK;
  int dev = -1;
  rmx_status st = check_device_arch(nullptr, &dev);
  if (st != RMX_OK) return st;
  const size_t esz = dtype_size(dtype);
  const size_t bytesE = size_t(B) * T * d * esz, bytesX = size_t(B) * T * D * esz;
  if ((st = check_dev(nullptr, E, bytesE, dev, "E")) != RMX_OK) return st;
  if ((st = check_dev(nullptr, Wp, size_t(T) * d * D * esz, dev, "Wp")) != RMX_OK) return st;
  if ((st = check_dev_opt(nullptr, bp, size_t(T) * D * esz, dev, "bp")) != RMX_OK) return st;
  if ((st = check_dev(nullptr, X, bytesX, dev, "X")) != RMX_OK) return st;
  const uintptr_t e = reinterpret_cast<uintptr_t>(E), x = reinterpret_cast<uintptr_t>(X);
  if (e < x + bytesX && x < e + bytesE) return fail(nullptr, RMX_ERR_INVALID_ARG, "E and X overlap");
  // token t is group t: A = E with rows T*d apart and groups d apart, C = X with rows T*D
  // apart and groups D apart
  GemmArgs g{};
  g.A = E;
  g.W = Wp;
  g.bias = bp;
  g.C = X;
  g.G = T;
  g.M = int(B);
  g.N = D;
  g.K = d;
  g.lda = int64_t(T) * d;
  g.sa = d;
  g.ldc = int64_t(T) * D;
  g.sc = D;
  hipError_t err = launch_gemm(dtype, EPI_BIAS, g, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(nullptr, RMX_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return RMX_OK;
}

rmx_status rmx_profile_enable(rmx_handle* h, int32_t enable) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  h->prof = enable != 0;
  return RMX_OK;
}

rmx_status rmx_profile_read(rmx_handle* h, double* total_ms, int64_t* launches, int64_t* dropped) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  for (auto& p : h->pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      h->total_ms[p.kind] += ms;
      h->launches[p.kind] += 1;
    } else {
      (void)hipGetLastError();
      ++h->dropped;
    }
    h->free_events.push_back(p.start);
    h->free_events.push_back(p.stop);
  }
  h->pending.clear();
  for (int i = 0; i < RMX_KERNEL_COUNT; ++i) {
    if (total_ms) total_ms[i] = h->total_ms[i];
    if (launches) launches[i] = h->launches[i];
  }
  if (dropped) *dropped = h->dropped;
  return RMX_OK;
}

rmx_status rmx_profile_reset(rmx_handle* h) {
  if (!h) return fail(nullptr, RMX_ERR_INVALID_ARG, "handle is NULL");
  double t[RMX_KERNEL_COUNT];
  int64_t n[RMX_KERNEL_COUNT];
  int64_t d;
  rmx_profile_read(h, t, n, &d);  // retire pending events
  for (int i = 0; i < RMX_KERNEL_COUNT; ++i) {
    h->total_ms[i] = 0.0;
    h->launches[i] = 0;
  }
  h->dropped = 0;
  return RMX_OK;
}

}  // extern "C"

// ------------------------------------------------------------ no-allocation forward
// rmx_block_forward_noalloc runs the dense forward with its workspace (S, the hidden H and
// the pre-LN2 rows Y, sized and laid out as a handle's for max_batch = B) carved out of
// `scratch`, a fixed array in device memory that the code object carries, so that the call
// allocates nothing.  Each device holds its own copy of the array; host code reaches it only
// through the device address hipGetSymbolAddress returns, taken once per device.
static __device__ __align__(256) unsigned char scratch[RMX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_noalloc_mutex;
std::atomic<unsigned char*> g_noalloc_ptr[NOALLOC_MAX_DEVICES];

// Once per device (the device current): the architecture check, the kernels' launch
// attributes and the device address of `scratch`.
rmx_status noalloc_device_scratch(int dev, unsigned char** out) {
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "device %d: the no-allocation path serves devices 0..%d", dev,
                NOALLOC_MAX_DEVICES - 1);
  unsigned char* p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    p = g_noalloc_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int d = -1;
      rmx_status st = check_device_arch(nullptr, &d);
      if (st != RMX_OK) return st;
      hipError_t e;
      if ((e = rows_init()) != hipSuccess || (e = gemm_init()) != hipSuccess)
        return fail(nullptr, RMX_ERR_HIP, "kernel set-up failed: %s", hipGetErrorString(e));
      void* q = nullptr;
      if ((e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch))) != hipSuccess || !q) {
        (void)hipGetLastError();
        return fail(nullptr, RMX_ERR_HIP, "device address of the scratch array: %s", hipGetErrorString(e));
      }
      p = static_cast<unsigned char*>(q);
      g_noalloc_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RMX_OK;
}

}  // namespace

extern "C" rmx_status rmx_block_forward_noalloc(const rmx_config* cfg, const void* X, int64_t B,
                                                 const rmx_weights* w, float* out, void* stream) {
  clear_error(nullptr);
  rmx_status st = validate_config(cfg);
  if (st != RMX_OK) return st;
  if (cfg->moe_experts != 0 || cfg->routing != RMX_ROUTING_MIX)
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "the no-allocation forward runs the dense Token Mixing block");
  if (!w) return fail(nullptr, RMX_ERR_INVALID_ARG, "weights is NULL");
  if (w->packed_mxfp8) return fail(nullptr, RMX_ERR_UNSUPPORTED, "the no-allocation forward runs bf16 or fp32 weights");
  if (B < 0) return fail(nullptr, RMX_ERR_INVALID_ARG, "B=%lld < 0", (long long)B);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "no HIP device");
  }
  unsigned char* base = nullptr;
  if ((st = noalloc_device_scratch(dev, &base)) != RMX_OK) return st;

  // the workspace of a handle created for max_batch = B
  rmx_handle tmp;
  tmp.cfg = *cfg;
  tmp.cfg.max_batch = B;
  tmp.device = dev;
  set_capabilities(&tmp);
  const size_t esz = dtype_size(cfg->dtype), T = cfg->T, D = cfg->D, kD = size_t(cfg->k) * cfg->D;
  const size_t prow = tmp.pk_capable ? T * size_t(pk_rows(B)) : T * size_t(B);
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t offH = up(prow * D * esz), offY = offH + up(prow * kD * esz), need = offY + T * size_t(B) * D * 4;
  if (need > RMX_NOALLOC_SCRATCH_BYTES)
    return fail(nullptr, RMX_ERR_UNSUPPORTED, "B=%lld needs %zu bytes of workspace; the no-allocation limit is %zu",
                (long long)B, need, size_t(RMX_NOALLOC_SCRATCH_BYTES));
  tmp.S = base;
  tmp.H = base + offH;
  tmp.Y = reinterpret_cast<float*>(base + offY);
  st = forward_impl(&tmp, X, B, w, cfg->L, cfg->k, out, nullptr, nullptr, nullptr, 0, stream);
  if (st != RMX_OK) g_thread_error = tmp.last_error;
  return st;
}
