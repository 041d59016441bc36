// Host-side launcher interface shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>

namespace mla {

// Raises the dynamic-LDS limit of kernels that need more than the default, once per device (the
// attribute belongs to the device's context): `done` holds one bit per device, set only after every
// hipFuncSetAttribute succeeded. Two threads making the first call on a device at once both set
// the attribute, which is harmless. Devices past the 32nd set it on every call.
struct LdsLimit {
  const void* fn;
  int bytes;
};
inline hipError_t ensure_lds_limit(std::atomic<uint32_t>& done, std::initializer_list<LdsLimit> fns) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = dev >= 0 && dev < 32 ? 1u << dev : 0u;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  for (const LdsLimit& f : fns) {
    e = hipFuncSetAttribute(f.fn, hipFuncAttributeMaxDynamicSharedMemorySize, f.bytes);
    if (e != hipSuccess) return e;
  }
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

struct LayerDims {
  int n_heads, d_nope, d_latent, d_rope, d_v;
  double rope_base;
  float softmax_scale;
};

// How one sequence's keys are cut into split-K chunks: chunk k covers keys
// [k * chunk_len, (k + 1) * chunk_len) of the visible range.
struct SplitPlan {
  int n_chunks;
  int chunk_len;
  // MFMA path only: how its workgroups take chunks (see attn_fast_plan), the grid's x extent and
  // the number of partial slots in the workspace
  int fast_mode;
  int fast_grid_x;
  int fast_slots;
};

constexpr int kMaxSplits = 256;

// Largest row (d_latent + d_rope) and d_nope the generic kernels accept.
constexpr int kGenericMaxRow = 1024;
constexpr int kGenericMaxNope = 256;

template <typename T>
hipError_t launch_rope_append_generic(const LayerDims& L, int batch, int n_new, const void* c_new, const void* k_new,
                                      void* cache, const int64_t* seq_off, const int32_t* len_before,
                                      hipStream_t stream);
template <typename T>
hipError_t launch_absorb_q_generic(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                   const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream);
template <typename T>
hipError_t launch_attn_generic(const LayerDims& L, int batch, int n_q, const void* q_packed, const void* cache,
                               const int64_t* seq_off, const int32_t* seq_len, const SplitPlan& plan, void* workspace,
                               float* z, float* lse, hipStream_t stream);
template <typename T>
hipError_t launch_out_proj_generic(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                   hipStream_t stream);

hipError_t launch_attn_merge(int n_rowheads, int n_chunks, int d_latent, const float* part_acc, const float* part_ml,
                             float* z, float* lse, hipStream_t stream);

// MFMA path for the DeepSeek-V2/V3 shape (H 128, d_latent 512, d_rope 64, bf16)
bool attn_fast_supported(const LayerDims& L);
void attn_fast_plan(int rows, int n_splits, int max_seq_len, SplitPlan* plan);
size_t attn_fast_workspace_bytes(const SplitPlan& plan, int rows);
// With defer_merge, a head-split plan's partials are left for launch_merge_out_proj.
hipError_t launch_attn_fast(const LayerDims& L, int batch, int n_q, const void* q_packed, const void* cache,
                            const int64_t* seq_off, const int32_t* seq_len, const SplitPlan& plan, void* workspace,
                            float* z, float* lse, hipStream_t stream, bool defer_merge = false);
bool attn_fast_is_hsplit(const SplitPlan& plan);
// The head-split plan's merge fused with the W_UV projection (rows < kGemmMinRows, bf16, the
// shape of proj_fast_supported): z, lse and o = W_UV z of every row, as the merge followed by
// launch_out_proj_fast would write them.
hipError_t launch_merge_out_proj(const LayerDims& L, int rows, const SplitPlan& plan, const void* workspace,
                                 const void* w_uv, float* z, float* lse, void* o, hipStream_t stream);

// The cache append of a decode step carried by the absorption launch (mla_decode_step): row
// r = b n_q + t is the new token t of sequence b, at position seq_len[b] - n_q + t; its latent is
// c_new[r] and its unrotated position key k_new[r]. vec as for the append kernel.
struct StepAppend {
  const void* c_new;
  const void* k_new;
  void* cache;
  const int64_t* seq_off;
  const int32_t* seq_len;
  int n_q;
  int vec;
};
bool append_vec_ok(const LayerDims& L, size_t elem_bytes, const void* c_new, const void* cache);

// GEMV-style projections for the DeepSeek-V2/V3 shape (H 128, d_nope = d_v 128, d_latent 512,
// d_rope 64, bf16). With `ap` the absorption launch also appends the step's new tokens (one
// extra workgroup column) and takes the query positions from ap->seq_len (q_pos NULL).
bool proj_fast_supported(const LayerDims& L);
hipError_t launch_absorb_q_fast(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream,
                                const StepAppend* ap = nullptr);
hipError_t launch_out_proj_fast(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                hipStream_t stream);
// MFMA GEMM forms of the same two projections (same shape), for many query rows at once
constexpr int kGemmMinRows = 16;

// y[r, n] = sum_k x[r, k] W[n, k] (linear.hip): the generic, matrix-vector or MFMA GEMM kernel by
// shape, dtype and alignment. Serves the optional W_O projection of mla_out_proj.
template <typename T>
hipError_t launch_linear(const void* x, int ldx, int M, int K, const void* w, int N, void* y, int ldy,
                         hipStream_t stream);
hipError_t launch_absorb_q_gemm(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream);
hipError_t launch_out_proj_gemm(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                hipStream_t stream);

// Upstream projections from the hidden state (linear.hip): workspace bytes, the kv side
// (W_DKV / W_KR -> RMSNorm -> RoPE -> cache rows) and the query side (W_DQ -> W_UQ / W_QR)
size_t project_workspace_bytes(const LayerDims& L, int n_rows, int d_q, int elem_bytes);
template <typename T>
hipError_t launch_project_kv_append(const LayerDims& L, int batch, int n_new, int d_model, const void* h,
                                    const void* w_dkv, const void* w_kr, const void* norm_w, float eps, int use_norm,
                                    void* cache, const int64_t* seq_off, const int32_t* len_before, void* workspace,
                                    hipStream_t stream);
template <typename T>
hipError_t launch_project_q(const LayerDims& L, int n_rows, int d_model, int d_q, const void* h, const void* w_dq,
                            const void* w_uq, const void* w_qr, void* q_nope, void* q_rope, void* workspace,
                            hipStream_t stream);
// both projections at once (mla_project_inputs): the kv side's float32 projection, then c_Q, in
// one workspace of project_inputs_workspace_bytes
size_t project_inputs_workspace_bytes(const LayerDims& L, int n_rows, int d_q, int elem_bytes);
template <typename T>
hipError_t launch_project_inputs(const LayerDims& L, int batch, int n_new, int d_model, int d_q, const void* h,
                                 const void* w_dkv, const void* w_kr, const void* norm_w, float eps, int use_norm,
                                 void* cache, const int64_t* seq_off, const int32_t* len_before, const void* w_dq,
                                 const void* w_uq, const void* w_qr, void* q_nope, void* q_rope, void* workspace,
                                 hipStream_t stream);

// Explicit (non-absorbed) prefill for the DeepSeek head shape (prefill_explicit.hip): K_C and V
// rebuilt by a GEMM over the cached latents (linear.hip), then multi-head attention with 192-wide
// keys; writes the heads' outputs o directly
hipError_t launch_kv_expand(int batch, int max_seq_len, int n_out, int d_latent, int row, const void* cache,
                            const int64_t* seq_off, const int32_t* seq_len, const void* w_uk, const void* w_uv,
                            void* kc, void* vv, hipStream_t stream);
bool prefill_explicit_supported(const LayerDims& L);
// From this many new query rows per sequence on, the explicit form measured faster than the
// absorbed one (absorb + latent attention + W_UV) on the DeepSeek head shape.
constexpr int kExplicitMinRows = 256;
size_t prefill_explicit_workspace_bytes(const LayerDims& L, int batch, int max_seq_len);
hipError_t launch_prefill_explicit(const LayerDims& L, int batch, int n_q, const void* q_nope, const void* q_rope,
                                   const void* cache, const int64_t* seq_off, const int32_t* seq_len, int max_seq_len,
                                   const void* w_uk, const void* w_uv, void* workspace, void* o, float* lse,
                                   hipStream_t stream);

// Position bookkeeping between decode steps (generic.hip)
hipError_t launch_decode_advance(int batch, int n_new, int32_t* len_before, int32_t* seq_len, int n_rows,
                                 int32_t* q_pos, hipStream_t stream);
// Append positions and query positions of a decode step from its key counts (generic.hip)
hipError_t launch_step_positions(const int32_t* seq_len, int batch, int n_q, int32_t* len_before, int32_t* q_pos,
                                 hipStream_t stream);

}  // namespace mla
