// C-ABI entry points of libmla: argument validation, split planning and dispatch.
// Nothing here allocates or synchronises; every launch goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/mla.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mla_status ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

mla_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shared checks on the layer description.
mla_status check_cfg(const mla_config* cfg, mla::LayerDims* L) {
  if (cfg == nullptr) return fail(MLA_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "cfg->reserved must be 0");
  if (cfg->n_heads < 1 || cfg->d_nope < 1 || cfg->d_latent < 1 || cfg->d_v < 1 || cfg->d_rope < 0)
    return fail(MLA_ERR_INVALID_ARG, "dims must be positive (d_rope >= 0): H=%d d_nope=%d d_latent=%d d_rope=%d d_v=%d",
                cfg->n_heads, cfg->d_nope, cfg->d_latent, cfg->d_rope, cfg->d_v);
  if (cfg->d_rope % 2 != 0) return fail(MLA_ERR_INVALID_ARG, "d_rope must be even, got %d", cfg->d_rope);
  if (cfg->dtype != MLA_F32 && cfg->dtype != MLA_BF16) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", cfg->dtype);
  if (!(cfg->softmax_scale > 0.0f) || !isfinite(cfg->softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!(cfg->rope_base > 0.0) || !isfinite(cfg->rope_base)) return fail(MLA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if ((int64_t)cfg->d_latent + cfg->d_rope > mla::kGenericMaxRow)
    return fail(MLA_ERR_UNSUPPORTED, "d_latent + d_rope = %d exceeds %d", cfg->d_latent + cfg->d_rope, mla::kGenericMaxRow);
  if (cfg->d_nope > mla::kGenericMaxNope)
    return fail(MLA_ERR_UNSUPPORTED, "d_nope = %d exceeds %d", cfg->d_nope, mla::kGenericMaxNope);
  L->n_heads = cfg->n_heads;
  L->d_nope = cfg->d_nope;
  L->d_latent = cfg->d_latent;
  L->d_rope = cfg->d_rope;
  L->d_v = cfg->d_v;
  L->rope_base = cfg->rope_base;
  L->softmax_scale = cfg->softmax_scale;
  return MLA_OK;
}

// Chunking of the keys for split-K. With n_splits = 0 the library picks: for the MFMA kernel about
// one workgroup per CU over the whole batch, but never chunks shorter than 256 keys (each chunk
// writes a 128 x 512 fp32 partial); for the generic kernel ~512 keys per chunk. At most 64.
mla_status plan_splits(int32_t max_seq_len, int32_t n_splits, int64_t rows, bool fast, mla::SplitPlan* plan) {
  if (n_splits < 0 || n_splits > mla::kMaxSplits)
    return fail(MLA_ERR_INVALID_ARG, "n_splits must be in [0, %d], got %d", mla::kMaxSplits, n_splits);
  int64_t n = n_splits;
  if (n == 0) {
    if (fast) {
      const int64_t by_cu = 256 / (rows > 0 ? rows : 1);
      const int64_t by_len = max_seq_len / 256;
      n = by_cu < by_len ? by_cu : by_len;
    } else {
      n = (max_seq_len + 511) / 512;
    }
    if (n > 64) n = 64;
    if (n < 1) n = 1;
  }
  if (n > max_seq_len) n = max_seq_len;
  plan->chunk_len = (int)((max_seq_len + n - 1) / n);
  plan->n_chunks = (max_seq_len + plan->chunk_len - 1) / plan->chunk_len;
  plan->fast_mode = plan->fast_grid_x = plan->fast_slots = 0;
  if (fast) mla::attn_fast_plan((int)rows, n_splits, max_seq_len, plan);
  return MLA_OK;
}

bool use_fast_attn(const mla_config* cfg, const mla::LayerDims& L) {
  return cfg->dtype == MLA_BF16 && mla::attn_fast_supported(L);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace: the generic kernels' partials ([row, head, chunk] x (d_latent + 2) floats) or, for the
// MFMA path, its partial slots; a shape that takes the MFMA path may still fall back to the
// generic kernels (unaligned pointers), so it is sized for both.
size_t attn_workspace_bytes(const mla::LayerDims& L, int batch, int n_q, const mla::SplitPlan& plan, bool fast) {
  size_t generic = 0;
  if (plan.n_chunks > 1) generic = (size_t)batch * n_q * L.n_heads * plan.n_chunks * ((size_t)L.d_latent + 2) * sizeof(float);
  const size_t fastb = fast ? mla::attn_fast_workspace_bytes(plan, batch * n_q) : 0;
  return generic > fastb ? generic : fastb;
}

// Launch choices shared by the single calls and mla_decode_step: the MFMA GEMM for many rows,
// the matrix-vector kernels for few, the generic kernels for other shapes, dtypes or alignments.
hipError_t absorb_dispatch(const mla_config* cfg, const mla::LayerDims& L, int n_rows, const void* q_nope,
                           const void* q_rope, const int32_t* q_pos, const void* w_uk, void* q_packed,
                           hipStream_t st) {
  const bool fast = cfg->dtype == MLA_BF16 && mla::proj_fast_supported(L) && aligned16(w_uk);
  if (fast && n_rows >= mla::kGemmMinRows && aligned16(q_nope) && aligned16(q_rope) && aligned16(q_packed))
    return mla::launch_absorb_q_gemm(L, n_rows, q_nope, q_rope, q_pos, w_uk, q_packed, st);
  if (fast) return mla::launch_absorb_q_fast(L, n_rows, q_nope, q_rope, q_pos, w_uk, q_packed, st);
  if (cfg->dtype == MLA_F32)
    return mla::launch_absorb_q_generic<float>(L, n_rows, q_nope, q_rope, q_pos, w_uk, q_packed, st);
  return mla::launch_absorb_q_generic<__bf16>(L, n_rows, q_nope, q_rope, q_pos, w_uk, q_packed, st);
}

// `defer` asks to leave a head-split plan's merge to launch_merge_out_proj; *deferred says whether
// it was (only on the MFMA path).
hipError_t attn_dispatch(const mla_config* cfg, const mla::LayerDims& L, int batch, int n_q, const void* q_packed,
                         const void* cache, const int64_t* seq_off, const int32_t* seq_len, const mla::SplitPlan& plan,
                         bool fast, void* workspace, float* z, float* lse, hipStream_t st, bool defer, bool* deferred) {
  if (deferred != nullptr) *deferred = false;
  if (fast && aligned16(q_packed) && aligned16(cache) && aligned16(z) && aligned16(workspace)) {
    const bool d = defer && mla::attn_fast_is_hsplit(plan);
    if (deferred != nullptr) *deferred = d;
    return mla::launch_attn_fast(L, batch, n_q, q_packed, cache, seq_off, seq_len, plan, workspace, z, lse, st, d);
  }
  if (cfg->dtype == MLA_F32)
    return mla::launch_attn_generic<float>(L, batch, n_q, q_packed, cache, seq_off, seq_len, plan, workspace, z, lse, st);
  return mla::launch_attn_generic<__bf16>(L, batch, n_q, q_packed, cache, seq_off, seq_len, plan, workspace, z, lse, st);
}

hipError_t out_proj_dispatch(const mla_config* cfg, const mla::LayerDims& L, int n_rows, const float* z,
                             const void* w_uv, void* o, hipStream_t st) {
  const bool fast = cfg->dtype == MLA_BF16 && mla::proj_fast_supported(L) && aligned16(w_uv) && aligned16(z);
  if (fast && n_rows >= mla::kGemmMinRows) return mla::launch_out_proj_gemm(L, n_rows, z, w_uv, o, st);
  if (fast) return mla::launch_out_proj_fast(L, n_rows, z, w_uv, o, st);
  if (cfg->dtype == MLA_F32) return mla::launch_out_proj_generic<float>(L, n_rows, z, w_uv, o, st);
  return mla::launch_out_proj_generic<__bf16>(L, n_rows, z, w_uv, o, st);
}

size_t round_up256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* mla_version(void) { return "mla 0.1.0 gfx950"; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not supported";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "unknown mla_status";
}

const char* mla_last_error(void) { return g_err; }

mla_status mla_rope_append(const mla_config* cfg, int32_t batch, int32_t n_new, const void* c_new,
                           const void* k_rope_new, void* cache, const int64_t* seq_off, const int32_t* len_before,
                           void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_new < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_new must be >= 0");
  if (batch == 0 || n_new == 0) return ok();
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
  if (!c_new || !cache || !seq_off || !len_before || (L.d_rope > 0 && !k_rope_new))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MLA_F32
                     ? mla::launch_rope_append_generic<float>(L, batch, n_new, c_new, k_rope_new, cache, seq_off, len_before, st)
                     : mla::launch_rope_append_generic<__bf16>(L, batch, n_new, c_new, k_rope_new, cache, seq_off, len_before, st);
  return from_hip(e, "mla_rope_append launch");
}

mla_status mla_absorb_q(const mla_config* cfg, int32_t n_rows, const void* q_nope, const void* q_rope,
                        const int32_t* q_pos, const void* w_uk, void* q_packed, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (n_rows == 0) return ok();
  if (L.n_heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "n_heads %d exceeds 65535", L.n_heads);
  if (!q_nope || !q_pos || !w_uk || !q_packed || (L.d_rope > 0 && !q_rope))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (n_rows > 65535 * 4) return fail(MLA_ERR_UNSUPPORTED, "n_rows %d exceeds %d", n_rows, 65535 * 4);
  return from_hip(absorb_dispatch(cfg, L, n_rows, q_nope, q_rope, q_pos, w_uk, q_packed, (hipStream_t)stream),
                  "mla_absorb_q launch");
}

size_t mla_decode_attn_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q, int32_t max_seq_len,
                                      int32_t n_splits) {
  mla::LayerDims L;
  if (check_cfg(cfg, &L) != MLA_OK) return 0;
  if (batch <= 0 || n_q <= 0 || max_seq_len < n_q) return 0;
  mla::SplitPlan plan;
  if (plan_splits(max_seq_len, n_splits, (int64_t)batch * n_q, use_fast_attn(cfg, L), &plan) != MLA_OK) return 0;
  return attn_workspace_bytes(L, batch, n_q, plan, use_fast_attn(cfg, L));
}

mla_status mla_decode_attn(const mla_config* cfg, int32_t batch, int32_t n_q, const void* q_packed, const void* cache,
                           const int64_t* seq_off, const int32_t* seq_len, int32_t max_seq_len, int32_t n_splits,
                           void* workspace, size_t workspace_bytes, float* z, float* lse, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_q < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_q must be >= 0");
  if (batch == 0 || n_q == 0) return ok();
  if (max_seq_len < n_q) return fail(MLA_ERR_INVALID_ARG, "max_seq_len (%d) must be >= n_q (%d)", max_seq_len, n_q);
  if ((int64_t)batch * n_q > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch * n_q exceeds 65535");
  if (L.n_heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "n_heads %d exceeds 65535", L.n_heads);
  if (!q_packed || !cache || !seq_off || !seq_len || !z) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  const bool fast = use_fast_attn(cfg, L);
  mla::SplitPlan plan;
  s = plan_splits(max_seq_len, n_splits, (int64_t)batch * n_q, fast, &plan);
  if (s != MLA_OK) return s;
  const size_t need = attn_workspace_bytes(L, batch, n_q, plan, fast);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  return from_hip(attn_dispatch(cfg, L, batch, n_q, q_packed, cache, seq_off, seq_len, plan, fast, workspace, z, lse,
                                (hipStream_t)stream, false, nullptr),
                  "mla_decode_attn launch");
}

mla_status mla_out_proj(const mla_config* cfg, int32_t n_rows, const float* z, const void* w_uv, void* o,
                        int32_t d_model, const void* w_o, void* u, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (d_model < 0) return fail(MLA_ERR_INVALID_ARG, "d_model must be >= 0, got %d", d_model);
  const bool with_w_o = d_model > 0;
  if (with_w_o != (w_o != nullptr) || with_w_o != (u != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "W_O projection: pass d_model > 0 with w_o and u, or d_model = 0 with both NULL");
  if (n_rows == 0) return ok();
  if (L.n_heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "n_heads %d exceeds 65535", L.n_heads);
  if (!z || !w_uv || !o) return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  hipStream_t st = (hipStream_t)stream;
  if (n_rows > 65535 * 4) return fail(MLA_ERR_UNSUPPORTED, "n_rows %d exceeds %d", n_rows, 65535 * 4);
  hipError_t e = out_proj_dispatch(cfg, L, n_rows, z, w_uv, o, st);
  if (e != hipSuccess || !with_w_o) return from_hip(e, "mla_out_proj launch");
  // u = W_O concat_i(o_i), from the o just written (same stream)
  const int K = L.n_heads * L.d_v;
  if ((int64_t)K > INT32_MAX / 8) return fail(MLA_ERR_UNSUPPORTED, "H * d_v too large");
  e = cfg->dtype == MLA_F32 ? mla::launch_linear<float>(o, K, n_rows, K, w_o, d_model, u, d_model, st)
                            : mla::launch_linear<__bf16>(o, K, n_rows, K, w_o, d_model, u, d_model, st);
  return from_hip(e, "mla_out_proj W_O launch");
}

size_t mla_decode_step_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q, int32_t max_seq_len,
                                      int32_t n_splits) {
  mla::LayerDims L;
  if (check_cfg(cfg, &L) != MLA_OK) return 0;
  if (batch <= 0 || n_q <= 0 || max_seq_len < n_q || (int64_t)batch * n_q > 65535) return 0;
  mla::SplitPlan plan;
  if (plan_splits(max_seq_len, n_splits, (int64_t)batch * n_q, use_fast_attn(cfg, L), &plan) != MLA_OK) return 0;
  // the attention's partials, then int32 append and query positions for the unfused launches
  return round_up256(attn_workspace_bytes(L, batch, n_q, plan, use_fast_attn(cfg, L))) +
         ((size_t)batch + (size_t)batch * n_q) * sizeof(int32_t);
}

}  // extern "C"

namespace {

// ---- Scratch of mla_decode_step_noalloc, for callers that cannot allocate (graph capture, tight
// serving loops). One array per GPU the library runs on, held until the process ends. In host code
// `scratch` is only a stand-in for the symbol, not a device address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to a kernel.
constexpr size_t kNoallocScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kNoallocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoallocMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

// device address of the current device's scratch array (resolved on the first call per device)
mla_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kNoallocMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "device %d: the scratch covers devices 0 .. %d", dev, kNoallocMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

// The body of mla_decode_step. With noalloc, the workspace is the library's own scratch array of
// workspace_bytes (its fixed size): a plan that needs more is rejected instead of reported as a
// short workspace.
mla_status decode_step_impl(const mla_config* cfg, int32_t batch, int32_t n_q, const void* c_new,
                            const void* k_rope_new, const void* q_nope, const void* q_rope, const void* w_uk,
                            const void* w_uv, void* cache, const int64_t* seq_off, const int32_t* seq_len,
                            int32_t max_seq_len, int32_t n_splits, void* workspace, size_t workspace_bytes,
                            void* q_packed, float* z, float* lse, void* o, void* stream, bool noalloc) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_q < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_q must be >= 0");
  if (batch == 0 || n_q == 0) return ok();
  if (max_seq_len < n_q) return fail(MLA_ERR_INVALID_ARG, "max_seq_len (%d) must be >= n_q (%d)", max_seq_len, n_q);
  if ((int64_t)batch * n_q > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch * n_q exceeds 65535");
  if (L.n_heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "n_heads %d exceeds 65535", L.n_heads);
  if (!c_new || !q_nope || !w_uk || !w_uv || !cache || !seq_off || !seq_len || !q_packed || !z || !o ||
      (L.d_rope > 0 && (!k_rope_new || !q_rope)))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  const int rows = batch * n_q;
  const bool fast = use_fast_attn(cfg, L);
  mla::SplitPlan plan;
  s = plan_splits(max_seq_len, n_splits, rows, fast, &plan);
  if (s != MLA_OK) return s;
  const size_t attn_bytes = round_up256(attn_workspace_bytes(L, batch, n_q, plan, fast));
  const size_t need = attn_bytes + ((size_t)batch + rows) * sizeof(int32_t);
  if (noalloc) {
    if (need > workspace_bytes)
      return fail(MLA_ERR_UNSUPPORTED, "this step needs %zu bytes of scratch, more than the %zu bytes the library holds",
                  need, workspace_bytes);
    s = noalloc_scratch(&workspace);
    if (s != MLA_OK) return s;
  }
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  // few rows of the DeepSeek shape: the append rides on the absorption launch, and the
  // head-split attention's merge on the W_UV launch (the same kernels and arithmetic as the
  // single calls, two launches fewer)
  const bool few = cfg->dtype == MLA_BF16 && mla::proj_fast_supported(L) && rows < mla::kGemmMinRows;
  if (few && aligned16(w_uk)) {
    const mla::StepAppend ap{c_new, k_rope_new, cache, seq_off, seq_len, n_q,
                             mla::append_vec_ok(L, sizeof(__bf16), c_new, cache) ? 1 : 0};
    e = mla::launch_absorb_q_fast(L, rows, q_nope, q_rope, nullptr, w_uk, q_packed, st, &ap);
    if (e != hipSuccess) return from_hip(e, "mla_decode_step append/absorb launch");
  } else {
    int32_t* len_before = (int32_t*)((char*)workspace + attn_bytes);
    int32_t* q_pos = len_before + batch;
    e = mla::launch_step_positions(seq_len, batch, n_q, len_before, q_pos, st);
    if (e == hipSuccess)
      e = cfg->dtype == MLA_F32
              ? mla::launch_rope_append_generic<float>(L, batch, n_q, c_new, k_rope_new, cache, seq_off, len_before, st)
              : mla::launch_rope_append_generic<__bf16>(L, batch, n_q, c_new, k_rope_new, cache, seq_off, len_before, st);
    if (e == hipSuccess) e = absorb_dispatch(cfg, L, rows, q_nope, q_rope, q_pos, w_uk, q_packed, st);
    if (e != hipSuccess) return from_hip(e, "mla_decode_step append/absorb launch");
  }
  bool deferred = false;
  e = attn_dispatch(cfg, L, batch, n_q, q_packed, cache, seq_off, seq_len, plan, fast, workspace, z, lse, st,
                    few && aligned16(w_uv), &deferred);
  if (e != hipSuccess) return from_hip(e, "mla_decode_step attention launch");
  e = deferred ? mla::launch_merge_out_proj(L, rows, plan, workspace, w_uv, z, lse, o, st)
               : out_proj_dispatch(cfg, L, rows, z, w_uv, o, st);
  return from_hip(e, "mla_decode_step output projection launch");
}

}  // namespace

extern "C" {

mla_status mla_decode_step(const mla_config* cfg, int32_t batch, int32_t n_q, const void* c_new, const void* k_rope_new,
                           const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv, void* cache,
                           const int64_t* seq_off, const int32_t* seq_len, int32_t max_seq_len, int32_t n_splits,
                           void* workspace, size_t workspace_bytes, void* q_packed, float* z, float* lse, void* o,
                           void* stream) {
  return decode_step_impl(cfg, batch, n_q, c_new, k_rope_new, q_nope, q_rope, w_uk, w_uv, cache, seq_off, seq_len,
                          max_seq_len, n_splits, workspace, workspace_bytes, q_packed, z, lse, o, stream, false);
}

mla_status mla_decode_step_noalloc(const mla_config* cfg, int32_t batch, int32_t n_q, const void* c_new,
                                   const void* k_rope_new, const void* q_nope, const void* q_rope, const void* w_uk,
                                   const void* w_uv, void* cache, const int64_t* seq_off, const int32_t* seq_len,
                                   int32_t max_seq_len, int32_t n_splits, void* q_packed, float* z, float* lse,
                                   void* o, void* stream) {
  // the scratch is resolved inside, once every argument and the plan's size have been checked
  return decode_step_impl(cfg, batch, n_q, c_new, k_rope_new, q_nope, q_rope, w_uk, w_uv, cache, seq_off, seq_len,
                          max_seq_len, n_splits, nullptr, kNoallocScratchBytes, q_packed, z, lse, o, stream, true);
}

size_t mla_project_workspace_size(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q) {
  mla::LayerDims L;
  if (check_cfg(cfg, &L) != MLA_OK) return 0;
  if (n_rows <= 0 || d_model <= 0 || d_q < 0) return 0;
  return mla::project_workspace_bytes(L, n_rows, d_q, cfg->dtype == MLA_F32 ? 4 : 2);
}

mla_status mla_project_kv_append(const mla_config* cfg, int32_t batch, int32_t n_new, int32_t d_model, const void* h,
                                 const void* w_dkv, const void* w_kr, const void* kv_norm_w, float kv_norm_eps,
                                 void* cache, const int64_t* seq_off, const int32_t* len_before, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_new < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_new must be >= 0");
  if (d_model < 1) return fail(MLA_ERR_INVALID_ARG, "d_model must be >= 1, got %d", d_model);
  if (kv_norm_w != nullptr && (!(kv_norm_eps >= 0.0f) || !isfinite(kv_norm_eps)))
    return fail(MLA_ERR_INVALID_ARG, "kv_norm_eps must be finite and >= 0");
  if (batch == 0 || n_new == 0) return ok();
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
  if ((int64_t)batch * n_new > (int64_t)INT32_MAX / 2) return fail(MLA_ERR_UNSUPPORTED, "batch * n_new too large");
  if (!h || !w_dkv || !cache || !seq_off || !len_before || (L.d_rope > 0 && !w_kr))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  const size_t need = mla::project_workspace_bytes(L, batch * n_new, 0, cfg->dtype == MLA_F32 ? 4 : 2);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  hipStream_t st = (hipStream_t)stream;
  const int use_norm = kv_norm_w != nullptr;
  hipError_t e = cfg->dtype == MLA_F32
                     ? mla::launch_project_kv_append<float>(L, batch, n_new, d_model, h, w_dkv, w_kr, kv_norm_w,
                                                            kv_norm_eps, use_norm, cache, seq_off, len_before,
                                                            workspace, st)
                     : mla::launch_project_kv_append<__bf16>(L, batch, n_new, d_model, h, w_dkv, w_kr, kv_norm_w,
                                                             kv_norm_eps, use_norm, cache, seq_off, len_before,
                                                             workspace, st);
  return from_hip(e, "mla_project_kv_append launch");
}

mla_status mla_project_q(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q, const void* h,
                         const void* w_dq, const void* w_uq, const void* w_qr, void* q_nope, void* q_rope,
                         void* workspace, size_t workspace_bytes, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (d_model < 1 || d_q < 0) return fail(MLA_ERR_INVALID_ARG, "need d_model >= 1 and d_q >= 0, got %d, %d", d_model, d_q);
  if ((d_q > 0) != (w_dq != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "pass w_dq exactly when d_q > 0 (query compression)");
  if (n_rows == 0) return ok();
  if (n_rows > 65535 * 4) return fail(MLA_ERR_UNSUPPORTED, "n_rows %d exceeds %d", n_rows, 65535 * 4);
  if ((int64_t)L.n_heads * (L.d_nope + L.d_rope) > (int64_t)INT32_MAX / 8)
    return fail(MLA_ERR_UNSUPPORTED, "query projection too wide");
  if (!h || !w_uq || !q_nope || (L.d_rope > 0 && (!w_qr || !q_rope)))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (d_q > 0) {
    const size_t need = mla::project_workspace_bytes(L, n_rows, d_q, cfg->dtype == MLA_F32 ? 4 : 2);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                  workspace ? "" : " (NULL)");
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MLA_F32
                     ? mla::launch_project_q<float>(L, n_rows, d_model, d_q, h, w_dq, w_uq, w_qr, q_nope, q_rope,
                                                    workspace, st)
                     : mla::launch_project_q<__bf16>(L, n_rows, d_model, d_q, h, w_dq, w_uq, w_qr, q_nope, q_rope,
                                                     workspace, st);
  return from_hip(e, "mla_project_q launch");
}

size_t mla_project_inputs_workspace_size(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q) {
  mla::LayerDims L;
  if (check_cfg(cfg, &L) != MLA_OK) return 0;
  if (n_rows <= 0 || d_model <= 0 || d_q < 0) return 0;
  return mla::project_inputs_workspace_bytes(L, n_rows, d_q, cfg->dtype == MLA_F32 ? 4 : 2);
}

mla_status mla_project_inputs(const mla_config* cfg, int32_t batch, int32_t n_new, int32_t d_model, int32_t d_q,
                              const void* h, const void* w_dkv, const void* w_kr, const void* kv_norm_w,
                              float kv_norm_eps, void* cache, const int64_t* seq_off, const int32_t* len_before,
                              const void* w_dq, const void* w_uq, const void* w_qr, void* q_nope, void* q_rope,
                              void* workspace, size_t workspace_bytes, void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_new < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_new must be >= 0");
  if (d_model < 1 || d_q < 0) return fail(MLA_ERR_INVALID_ARG, "need d_model >= 1 and d_q >= 0, got %d, %d", d_model, d_q);
  if ((d_q > 0) != (w_dq != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "pass w_dq exactly when d_q > 0 (query compression)");
  if (kv_norm_w != nullptr && (!(kv_norm_eps >= 0.0f) || !isfinite(kv_norm_eps)))
    return fail(MLA_ERR_INVALID_ARG, "kv_norm_eps must be finite and >= 0");
  if (batch == 0 || n_new == 0) return ok();
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
  const int64_t rows = (int64_t)batch * n_new;
  if (rows > 65535 * 4) return fail(MLA_ERR_UNSUPPORTED, "batch * n_new = %lld exceeds %d", (long long)rows, 65535 * 4);
  if ((int64_t)L.n_heads * (L.d_nope + L.d_rope) > (int64_t)INT32_MAX / 8)
    return fail(MLA_ERR_UNSUPPORTED, "query projection too wide");
  if (!h || !w_dkv || !cache || !seq_off || !len_before || !w_uq || !q_nope ||
      (L.d_rope > 0 && (!w_kr || !w_qr || !q_rope)))
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  const size_t need = mla::project_inputs_workspace_bytes(L, (int)rows, d_q, cfg->dtype == MLA_F32 ? 4 : 2);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  const int use_norm = kv_norm_w != nullptr;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = cfg->dtype == MLA_F32
                     ? mla::launch_project_inputs<float>(L, batch, n_new, d_model, d_q, h, w_dkv, w_kr, kv_norm_w,
                                                         kv_norm_eps, use_norm, cache, seq_off, len_before, w_dq, w_uq,
                                                         w_qr, q_nope, q_rope, workspace, st)
                     : mla::launch_project_inputs<__bf16>(L, batch, n_new, d_model, d_q, h, w_dkv, w_kr, kv_norm_w,
                                                          kv_norm_eps, use_norm, cache, seq_off, len_before, w_dq, w_uq,
                                                          w_qr, q_nope, q_rope, workspace, st);
  return from_hip(e, "mla_project_inputs launch");
}

size_t mla_prefill_explicit_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q, int32_t max_seq_len) {
  mla::LayerDims L;
  if (check_cfg(cfg, &L) != MLA_OK) return 0;
  if (batch <= 0 || n_q <= 0 || max_seq_len < n_q) return 0;
  if (cfg->dtype != MLA_BF16 || !mla::prefill_explicit_supported(L)) return 0;
  return mla::prefill_explicit_workspace_bytes(L, batch, max_seq_len);
}

mla_status mla_prefill_explicit(const mla_config* cfg, int32_t batch, int32_t n_q, const void* q_nope,
                                const void* q_rope, const void* cache, const int64_t* seq_off, const int32_t* seq_len,
                                int32_t max_seq_len, const void* w_uk, const void* w_uv, void* workspace,
                                size_t workspace_bytes, void* o, float* lse, int32_t d_model, const void* w_o, void* u,
                                void* stream) {
  mla::LayerDims L;
  mla_status s = check_cfg(cfg, &L);
  if (s != MLA_OK) return s;
  if (batch < 0 || n_q < 0) return fail(MLA_ERR_INVALID_ARG, "batch and n_q must be >= 0");
  if (d_model < 0) return fail(MLA_ERR_INVALID_ARG, "d_model must be >= 0, got %d", d_model);
  const bool with_w_o = d_model > 0;
  if (with_w_o != (w_o != nullptr) || with_w_o != (u != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "W_O projection: pass d_model > 0 with w_o and u, or d_model = 0 with both NULL");
  if (batch == 0 || n_q == 0) return ok();
  if (max_seq_len < n_q) return fail(MLA_ERR_INVALID_ARG, "max_seq_len (%d) must be >= n_q (%d)", max_seq_len, n_q);
  if (cfg->dtype != MLA_BF16 || !mla::prefill_explicit_supported(L))
    return fail(MLA_ERR_UNSUPPORTED, "the explicit prefill covers bf16 with d_nope = d_v = 128, d_rope = 64, d_latent = 512");
  if ((int64_t)batch * L.n_heads * ((n_q + 127) / 128) > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "batch * heads * query blocks too large");
  if ((int64_t)max_seq_len > 65535 * 128) return fail(MLA_ERR_UNSUPPORTED, "max_seq_len %d too large", max_seq_len);
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
  // the key/value rebuild runs 2 H column tiles of 128 in its grid's second dimension
  if (L.n_heads > 32767) return fail(MLA_ERR_UNSUPPORTED, "n_heads %d exceeds 32767", L.n_heads);
  if (!q_nope || !q_rope || !cache || !seq_off || !seq_len || !w_uk || !w_uv || !o)
    return fail(MLA_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(cache) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(o) || !aligned16(workspace) || (with_w_o && (!aligned16(w_o) || !aligned16(u))))
    return fail(MLA_ERR_INVALID_ARG, "tensors of the explicit prefill must be 16-byte aligned");
  if (with_w_o && (int64_t)L.n_heads * L.d_v > INT32_MAX / 8) return fail(MLA_ERR_UNSUPPORTED, "H * d_v too large");
  const size_t need = mla::prefill_explicit_workspace_bytes(L, batch, max_seq_len);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                workspace ? "" : " (NULL)");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = mla::launch_prefill_explicit(L, batch, n_q, q_nope, q_rope, cache, seq_off, seq_len, max_seq_len, w_uk,
                                              w_uv, workspace, o, lse, st);
  if (e != hipSuccess || !with_w_o) return from_hip(e, "mla_prefill_explicit launch");
  // u = W_O concat_i(o_i), from the o just written (same stream), as mla_out_proj does
  const int K = L.n_heads * L.d_v;
  e = mla::launch_linear<__bf16>(o, K, batch * n_q, K, w_o, d_model, u, d_model, st);
  return from_hip(e, "mla_prefill_explicit W_O launch");
}

int32_t mla_prefill_prefers_explicit(const mla_config* cfg, int32_t batch, int32_t n_q, int32_t max_seq_len) {
  mla::LayerDims L;
  if (cfg == nullptr || check_cfg(cfg, &L) != MLA_OK) return 0;
  if (batch <= 0 || n_q <= 0 || max_seq_len < n_q) return 0;
  if (cfg->dtype != MLA_BF16 || !mla::prefill_explicit_supported(L)) return 0;
  return n_q >= mla::kExplicitMinRows ? 1 : 0;
}

mla_status mla_decode_advance(int32_t batch, int32_t n_new, int32_t* len_before, int32_t* seq_len, int32_t n_rows,
                              int32_t* q_pos, void* stream) {
  if (batch < 0 || n_rows < 0 || n_new < 0) return fail(MLA_ERR_INVALID_ARG, "batch, n_new and n_rows must be >= 0");
  const bool any_b = batch > 0 && (len_before != nullptr || seq_len != nullptr);
  const bool any_q = n_rows > 0 && q_pos != nullptr;
  if (n_new == 0 || (!any_b && !any_q)) return ok();
  hipError_t e = mla::launch_decode_advance(any_b ? batch : 0, n_new, len_before, seq_len, any_q ? n_rows : 0, q_pos,
                                            (hipStream_t)stream);
  return from_hip(e, "mla_decode_advance launch");
}

}  // extern "C"
