/*
 * libmla — absorbed Multi-head Latent Attention decode with decoupled RoPE, for MI355X (gfx950).
 *
 * The four compute calls follow the inference flow of one new token in
 * "Decoupled RoPE · MLA Part 2" (agent.namiai.tech), §5: append the token's latent c and its
 * rotated position key to the cache, absorb the content query through W_UK, score every cached
 * row with q~·c + q_R·k_R, softmax, sum the latents, and project once through W_UV.
 *
 * Conventions shared by every call
 *  - Ownership: every data pointer is device memory allocated and owned by the caller. The
 *    library never allocates, frees or synchronises; each call only enqueues kernels on
 *    `stream` (a hipStream_t; NULL means the legacy default stream) and returns.
 *  - Layout: row-major and contiguous. Weights keep the nn.Linear [out, in] layout, viewed per
 *    head ("从零理解 MLA", section "矩阵吸收" code note on the weight view).
 *  - Storage dtype: `cfg->dtype` is the dtype of the cache, the weights, q_nope/q_rope,
 *    q_packed and o. Latent outputs z and lse are always float32. Arithmetic accumulates in
 *    float32; RoPE angles are formed and reduced in float64.
 *  - Cache: token p of sequence b is row (seq_off[b] + p); a row is
 *    [c (d_latent) ; RoPE_p(k_R) (d_rope)], latent first ("从零理解 MLA", section "解耦 RoPE",
 *    absorbed_step, where the cached entry is the concatenation of c_kv and the rotated k_r).
 *  - RoPE: consecutive pairs (2j, 2j+1) of a position vector at position p are turned by
 *    p·theta_j, theta_j = rope_base^(-2j/d_rope) ("Decoupled RoPE · MLA Part 2", §4 and §7).
 *  - Device metadata (seq_off, len_before, seq_len, q_pos) is trusted: the caller guarantees
 *    slab capacity, 0 < n_q <= seq_len[b] <= max_seq_len, and positions within int32.
 *  - Errors: arguments are validated before anything is launched; a failing check returns a
 *    status, launches nothing and writes nothing. A failed launch returns MLA_ERR_HIP.
 *    mla_last_error() gives the calling thread's detail text for the last non-OK status.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Empty work (batch == 0, n_new == 0, n_rows == 0) is valid and launches nothing.
 *  - Outputs must not alias inputs; only `cache` is read-write.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape, bad scale/base */
  MLA_ERR_UNSUPPORTED = 2, /* dims or dtype outside what the compiled kernels cover */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than mla_decode_attn_workspace_size */
  MLA_ERR_HIP = 4          /* a HIP runtime call or launch failed; see mla_last_error() */
} mla_status;

typedef enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Shape and numeric parameters of one MLA layer. 40 bytes, no padding surprises. */
typedef struct mla_config {
  int32_t n_heads;     /* H: attention heads (128 for DeepSeek-V2/V3) */
  int32_t d_nope;      /* per-head content query/key width d_h (128) */
  int32_t d_latent;    /* latent width d_c (512) */
  int32_t d_rope;      /* decoupled position width d_R (64); even, may be 0 */
  int32_t d_v;         /* per-head value width (128) */
  int32_t dtype;       /* mla_dtype of stored tensors */
  double rope_base;    /* RoPE base (10000); > 0 */
  float softmax_scale; /* score scale, 1/sqrt(d_nope + d_rope) in the pages' models; > 0 */
  int32_t reserved;    /* must be 0 */
} mla_config;

/* Library version string, e.g. "mla 0.1.0 gfx950". */
const char* mla_version(void);

/* Static text for a status code. */
const char* mla_status_string(mla_status status);

/* Detail text of the calling thread's last non-OK status ("" if none). */
const char* mla_last_error(void);

/*
 * mla_rope_append — cache append ("Decoupled RoPE · MLA Part 2", §3.4: a key's position part is
 * rotated once, when the token is first computed, and stored rotated; §5 steps 2–3).
 *
 * For b < batch and i < n_new, with p = len_before[b] + i:
 *   cache[seq_off[b] + p] = [ c_new[b, i, :] ; RoPE_p(k_rope_new[b, i, :]) ]
 *  c_new       [batch, n_new, d_latent]  storage dtype, device
 *  k_rope_new  [batch, n_new, d_rope]    storage dtype, device, unrotated
 *  cache       rows of d_latent + d_rope storage-dtype elements, device, written
 *  seq_off     int64 [batch] device: first cache row of each sequence's slab
 *  len_before  int32 [batch] device: tokens already cached (position of the first new token)
 */
mla_status mla_rope_append(const mla_config* cfg, int32_t batch, int32_t n_new,
                           const void* c_new, const void* k_rope_new, void* cache,
                           const int64_t* seq_off, const int32_t* len_before, void* stream);

/*
 * mla_absorb_q — query absorption ("从零理解 MLA", section "矩阵吸收": the content logit
 * q_C·(W_UK,i c) equals (W_UK,i^T q_C)·c; "Decoupled RoPE · MLA Part 2", §5 step 4).
 *
 * For r < n_rows, head i < H:
 *   q_packed[r, i, 0:d_latent]               = W_UK,i^T q_nope[r, i, :]
 *   q_packed[r, i, d_latent:d_latent+d_rope] = RoPE_{q_pos[r]}(q_rope[r, i, :])
 *  q_nope    [n_rows, H, d_nope]   storage dtype, device
 *  q_rope    [n_rows, H, d_rope]   storage dtype, device, unrotated
 *  q_pos     int32 [n_rows] device: position of each query row
 *  w_uk      [H, d_nope, d_latent] storage dtype, device (nn.Linear(d_latent, H*d_nope).weight)
 *  q_packed  [n_rows, H, d_latent + d_rope] storage dtype, device, written
 */
mla_status mla_absorb_q(const mla_config* cfg, int32_t n_rows, const void* q_nope, const void* q_rope,
                        const int32_t* q_pos, const void* w_uk, void* q_packed, void* stream);

/*
 * Bytes of device workspace mla_decode_attn needs for these sizes (0 when no split-K partials
 * are needed). n_splits = 0 selects the library's choice. Returns 0 for invalid arguments.
 */
size_t mla_decode_attn_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q,
                                      int32_t max_seq_len, int32_t n_splits);

/*
 * mla_decode_attn — latent attention over the packed cache (scores, mask, softmax, latent sum;
 * "Decoupled RoPE · MLA Part 2", §3.2 and §5 steps 4–5; value = the latent part of the same
 * cached row, "从零理解 MLA", section "矩阵吸收").
 *
 * Query row t of sequence b sits at position seq_len[b] - n_q + t and sees keys
 * j <= seq_len[b] - n_q + t (the causal mask with diagonal offset S - L, "从零理解 MLA",
 * section "KV Cache"); for decode (n_q = 1) that is every cached key including itself.
 *   s_j   = softmax_scale * <q_packed[b, t, i, :], cache[seq_off[b] + j, :]>   (d_latent + d_rope)
 *   z     = sum_j softmax(s)_j * cache[seq_off[b] + j, 0:d_latent]
 *   lse   = ln sum_j exp(s_j)
 *  q_packed  [batch, n_q, H, d_latent + d_rope] storage dtype, device
 *  cache     packed rows (see top), device, read
 *  seq_off   int64 [batch] device;  seq_len int32 [batch] device: keys incl. the n_q new ones
 *  max_seq_len  host upper bound of seq_len (grid sizing)
 *  n_splits  split-K chunks per sequence (0 = library choice); results do not depend on it
 *            beyond float32 summation order
 *  workspace device scratch of at least mla_decode_attn_workspace_size(...) bytes (may be
 *            NULL when that size is 0); contents need no initialisation
 *  z         float32 [batch, n_q, H, d_latent] device, written
 *  lse       float32 [batch, n_q, H] device, written; may be NULL
 */
mla_status mla_decode_attn(const mla_config* cfg, int32_t batch, int32_t n_q, const void* q_packed,
                           const void* cache, const int64_t* seq_off, const int32_t* seq_len,
                           int32_t max_seq_len, int32_t n_splits, void* workspace,
                           size_t workspace_bytes, float* z, float* lse, void* stream);

/*
 * mla_out_proj — output projection in latent space ("从零理解 MLA", section "矩阵吸收",
 * output-side equation o_i = W_UV,i z_i; "Decoupled RoPE · MLA Part 2", §5 step 5).
 *
 * For r < n_rows, head i:  o[r, i, :] = W_UV,i z[r, i, :]
 *  z     float32 [n_rows, H, d_latent] device
 *  w_uv  [H, d_v, d_latent] storage dtype, device (nn.Linear(d_latent, H*d_v).weight)
 *  o     [n_rows, H, d_v] storage dtype, device, written
 *  d_model, w_o, u: optional layer output u = W_O concat_i(o_i) ("Decoupled RoPE · MLA Part 2",
 *        §5 step 5 and the output line of the §7 forward pass; "从零理解 MLA", section "矩阵吸收").
 *        d_model = 0 with w_o = u = NULL skips it. With d_model > 0:
 *          w_o  [d_model, H * d_v] storage dtype, device (nn.Linear(H*d_v, d_model).weight); the
 *               concatenation is head-major: column i * d_v + v multiplies o[r, i, v]
 *          u    [n_rows, d_model] storage dtype, device, written (fp32 accumulation over the o
 *               this call stores, rounded once)
 *        Any other combination returns MLA_ERR_INVALID_ARG.
 */
mla_status mla_out_proj(const mla_config* cfg, int32_t n_rows, const float* z, const void* w_uv,
                        void* o, int32_t d_model, const void* w_o, void* u, void* stream);

/*
 * ---- The four calls as one decode step.
 *
 * Bytes of device workspace mla_decode_step needs (the attention's split-K partials plus
 * 4 (batch + batch * n_q) bytes of positions). 0 for invalid arguments.
 */
size_t mla_decode_step_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q,
                                      int32_t max_seq_len, int32_t n_splits);

/*
 * mla_decode_step — one step of the inference flow of "Decoupled RoPE · MLA Part 2", §5 (steps
 * 2–5): append the n_q new tokens of every sequence, absorb their queries, attend, project
 * through W_UV. The positions come from seq_len, which already counts the new tokens: token t of
 * sequence b (row r = b * n_q + t) sits at position p = seq_len[b] - n_q + t. The results are
 * those of the four single calls in order:
 *   mla_rope_append(cfg, batch, n_q, c_new, k_rope_new, cache, seq_off, len_before = seq_len - n_q)
 *   mla_absorb_q(cfg, batch * n_q, q_nope, q_rope, q_pos = p of each row, w_uk, q_packed)
 *   mla_decode_attn(cfg, batch, n_q, q_packed, cache, seq_off, seq_len, max_seq_len, n_splits, ..., z, lse)
 *   mla_out_proj(cfg, batch * n_q, z, w_uv, o, 0, NULL, NULL)
 * the cache rows and q_packed bit for bit, z, lse and o bit for bit except where the step fuses
 * the split-K merge: for few rows of the DeepSeek shape in bf16 (batch * n_q < 16) it needs two
 * launches fewer, as the append rides on the absorption's launch and the head-split attention's
 * merge on the projection's; z and lse then differ from mla_decode_attn's only by float32
 * summation order, and o by the one bf16 rounding that follows.
 *  c_new [batch, n_q, d_latent], k_rope_new [batch, n_q, d_rope] (unrotated), q_nope
 *        [batch * n_q, H, d_nope], q_rope [batch * n_q, H, d_rope] (unrotated), w_uk, w_uv: as for
 *        the single calls (storage dtype, device)
 *  cache, seq_off, seq_len, max_seq_len, n_splits: as for mla_decode_attn; cache is written
 *  workspace  >= mla_decode_step_workspace_size(...) bytes, device; no initialisation
 *  q_packed [batch * n_q, H, d_latent + d_rope], z float32 [batch, n_q, H, d_latent], o
 *        [batch * n_q, H, d_v]: written (q_packed and z are the intermediate results of the
 *        single calls); lse float32 [batch, n_q, H] written, may be NULL
 * Errors and limits: those of the four single calls.
 */
mla_status mla_decode_step(const mla_config* cfg, int32_t batch, int32_t n_q, const void* c_new,
                           const void* k_rope_new, const void* q_nope, const void* q_rope,
                           const void* w_uk, const void* w_uv, void* cache, const int64_t* seq_off,
                           const int32_t* seq_len, int32_t max_seq_len, int32_t n_splits,
                           void* workspace, size_t workspace_bytes, void* q_packed, float* z,
                           float* lse, void* o, void* stream);

/*
 * mla_decode_step_noalloc — mla_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Same arguments,
 * results, kernels and errors as mla_decode_step, minus the workspace: the split-K partials and the
 * step's positions go to a scratch array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on (a static device array, resolved once per device on the first call made
 * with that device current, and held until the process ends). The call allocates and frees
 * nothing.
 *  - The array of the current device (hipGetDevice) is used: `stream` must belong to that device.
 *  - A step whose workspace (mla_decode_step_workspace_size) exceeds MLA_NOALLOC_SCRATCH_BYTES
 *    returns MLA_ERR_UNSUPPORTED and launches nothing.
 *  - No part of the array needs to start at zero: every word the step's kernels read is written
 *    earlier in the same step. The array keeps the last call's contents.
 *  - All calls on one GPU share its array: calls that overlap in time on one GPU (different
 *    streams, or different threads without ordering) race and give wrong results. Order them on
 *    one stream.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_step_noalloc(const mla_config* cfg, int32_t batch, int32_t n_q, const void* c_new,
                                   const void* k_rope_new, const void* q_nope, const void* q_rope,
                                   const void* w_uk, const void* w_uv, void* cache, const int64_t* seq_off,
                                   const int32_t* seq_len, int32_t max_seq_len, int32_t n_splits,
                                   void* q_packed, float* z, float* lse, void* o, void* stream);

/*
 * ---- Upstream projections: from the hidden state h to the inputs of the calls above.
 *
 * Bytes of device workspace mla_project_kv_append (d_q = 0) or mla_project_q (its d_q) needs
 * for n_rows tokens; take the larger of the two to share one buffer. 0 for invalid arguments.
 */
size_t mla_project_workspace_size(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q);

/*
 * mla_project_kv_append — cache side of the layer from h ("Decoupled RoPE · MLA Part 2", §5
 * steps 2–3: the latent and the position key both come from h, and the key is rotated once when
 * stored; "构建DeepSeek-V3：MLA 架构", step 1: the compressed latent is RMS-normalised,
 * c_KV = RMSNorm(W_dkv x), with the RMSNorm of "hands-on DeepSeek MLA").
 *
 * For b < batch, i < n_new, with x = h[b, i, :] and p = len_before[b] + i:
 *   c    = W_DKV x, then, when kv_norm_w != NULL, c = kv_norm_w * c / sqrt(mean(c^2) + kv_norm_eps)
 *   k_R  = W_KR x
 *   cache[seq_off[b] + p] = [ c ; RoPE_p(k_R) ]        (as mla_rope_append stores it)
 *  h          [batch, n_new, d_model]  storage dtype, device
 *  w_dkv      [d_latent, d_model]      storage dtype, device (nn.Linear(d_model, d_latent).weight)
 *  w_kr       [d_rope, d_model]        storage dtype, device; may be NULL when d_rope = 0
 *  kv_norm_w  [d_latent] storage dtype, device, the RMSNorm gain; NULL = no normalisation
 *  kv_norm_eps  >= 0, finite (1e-6 in the pages' RMSNorm); ignored without kv_norm_w
 *  cache, seq_off, len_before  as for mla_rope_append
 *  workspace  device scratch of at least mla_project_workspace_size(cfg, batch * n_new, d_model, 0)
 *             bytes (float32 projections before the norm and the rotation); no initialisation
 * Products accumulate in float32, the norm is taken in float32, the rotation in float64, and each
 * stored value is rounded once.
 */
mla_status mla_project_kv_append(const mla_config* cfg, int32_t batch, int32_t n_new, int32_t d_model,
                                 const void* h, const void* w_dkv, const void* w_kr, const void* kv_norm_w,
                                 float kv_norm_eps, void* cache, const int64_t* seq_off,
                                 const int32_t* len_before, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * mla_project_q — query side of the layer from h ("从零理解 MLA", sections "查询压缩" and
 * "解耦 RoPE": the content query comes from the compressed c_Q, and so does the position query;
 * "构建DeepSeek-V3：MLA 架构", q_rope = RoPE(W_qr c_Q), with no norm on c_Q).
 *
 * With query compression (d_q > 0):  c_Q = W_DQ h;  q_nope = W_UQ c_Q;  q_rope = W_QR c_Q.
 * Without (d_q = 0, w_dq = NULL):     q_nope = W_UQ h;  q_rope = W_QR h (W_UQ is then W_Q).
 * The outputs are exactly mla_absorb_q's inputs: q_rope is NOT rotated here.
 *  h        [n_rows, d_model] storage dtype, device
 *  w_dq     [d_q, d_model] storage dtype, device, or NULL when d_q = 0
 *  w_uq     [H * d_nope, d_q or d_model] storage dtype, device (rows head-major)
 *  w_qr     [H * d_rope, d_q or d_model] storage dtype, device; may be NULL when d_rope = 0
 *  q_nope   [n_rows, H, d_nope] storage dtype, device, written
 *  q_rope   [n_rows, H, d_rope] storage dtype, device, written; may be NULL when d_rope = 0
 *  workspace  device scratch of at least mla_project_workspace_size(cfg, n_rows, d_model, d_q)
 *           bytes when d_q > 0 (c_Q, rounded once to the storage dtype); ignored when d_q = 0
 */
mla_status mla_project_q(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q,
                         const void* h, const void* w_dq, const void* w_uq, const void* w_qr,
                         void* q_nope, void* q_rope, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Bytes of device workspace mla_project_inputs needs for n_rows tokens: the kv side's float32
 * projection and c_Q side by side. 0 for invalid arguments.
 */
size_t mla_project_inputs_workspace_size(const mla_config* cfg, int32_t n_rows, int32_t d_model, int32_t d_q);

/*
 * mla_project_inputs — both projections of a layer's input h in one call: exactly
 *   mla_project_kv_append(cfg, batch, n_new, d_model, h, w_dkv, w_kr, kv_norm_w, kv_norm_eps, cache,
 *                         seq_off, len_before, ...)
 *   mla_project_q(cfg, batch * n_new, d_model, d_q, h, w_dq, w_uq, w_qr, q_nope, q_rope, ...)
 * with the same arguments, layouts and limits (the passages cited there), h read as
 * [batch * n_new, d_model] for the query side. For fewer than 16 rows of bf16 (16-byte aligned
 * tensors, d_model and d_q multiples of 8) it takes two launches instead of four: h is read once
 * for W_DKV, W_KR and W_DQ, and the latent's RMSNorm and the key's rotation ride on the W_UQ / W_QR
 * launch. The products are the same up to float32 summation order.
 *  workspace  >= mla_project_inputs_workspace_size(cfg, batch * n_new, d_model, d_q) bytes, device;
 *             no initialisation
 */
mla_status mla_project_inputs(const mla_config* cfg, int32_t batch, int32_t n_new, int32_t d_model, int32_t d_q,
                              const void* h, const void* w_dkv, const void* w_kr, const void* kv_norm_w,
                              float kv_norm_eps, void* cache, const int64_t* seq_off,
                              const int32_t* len_before, const void* w_dq, const void* w_uq,
                              const void* w_qr, void* q_nope, void* q_rope, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * ---- Explicit (non-absorbed) prefill: the same attention output o for many query rows at once.
 *
 * Bytes of device workspace mla_prefill_explicit needs (the rebuilt content keys and values:
 * 2 * batch * max_seq_len * H * 128 bf16). 0 for invalid arguments or a shape the call does not
 * cover.
 */
size_t mla_prefill_explicit_workspace_size(const mla_config* cfg, int32_t batch, int32_t n_q,
                                           int32_t max_seq_len);

/*
 * mla_prefill_explicit — attention of n_q new query rows per sequence in the non-absorbed form
 * ("Decoupled RoPE · MLA Part 2", §2.1 and §3.2: per head the content key W_UK,i c and the value
 * W_UV,i c are rebuilt from the cached latent, the shared rotated position key is concatenated to
 * the content key, q = [q_nope ; RoPE(q_rope)]; "从零理解 MLA", the non-absorbed forward). For long
 * query chunks this needs 2 H (192 + 128) flops per (row, key) instead of the absorbed 2 H (576 + 512).
 *
 * Same mask and positions as mla_decode_attn (query row t of sequence b at position
 * seq_len[b] - n_q + t sees keys j <= seq_len[b] - n_q + t); the cache must already hold the rows of
 * all seq_len[b] tokens (mla_rope_append). For each (b, t, head i):
 *   s_j  = softmax_scale * ( q_nope[b,t,i] . (W_UK,i c_j) + RoPE_pos(q_rope[b,t,i]) . k_R,j )
 *   o    = sum_j softmax(s)_j (W_UV,i c_j);   lse = ln sum_j exp(s_j)
 * which equals mla_out_proj(mla_decode_attn(mla_absorb_q(...))) up to rounding.
 *  q_nope   [batch, n_q, H, 128] bf16, device;  q_rope [batch, n_q, H, 64] bf16, device, unrotated
 *  cache, seq_off, seq_len, max_seq_len   as for mla_decode_attn
 *  w_uk     [H, 128, 512] bf16, device;  w_uv [H, 128, 512] bf16, device
 *  workspace  >= mla_prefill_explicit_workspace_size(...) bytes, device; no initialisation
 *  o        [batch, n_q, H, 128] bf16, device, written
 *  lse      float32 [batch, n_q, H], device, written; may be NULL
 *  d_model, w_o, u: optional layer output u = W_O concat_i(o_i), exactly as for mla_out_proj
 *           (d_model = 0 with w_o = u = NULL skips it; w_o [d_model, H * 128], u [batch * n_q, d_model]
 *           bf16, 16-byte aligned)
 * Covers bf16 with d_nope = d_v = 128, d_rope = 64, d_latent = 512 (any head count); anything
 * else returns MLA_ERR_UNSUPPORTED. All tensors must be 16-byte aligned. Keys and values are
 * rounded once to bf16 when rebuilt; scores, softmax and sums accumulate in float32.
 */
mla_status mla_prefill_explicit(const mla_config* cfg, int32_t batch, int32_t n_q, const void* q_nope,
                                const void* q_rope, const void* cache, const int64_t* seq_off,
                                const int32_t* seq_len, int32_t max_seq_len, const void* w_uk,
                                const void* w_uv, void* workspace, size_t workspace_bytes, void* o,
                                float* lse, int32_t d_model, const void* w_o, void* u, void* stream);

/*
 * mla_prefill_prefers_explicit — which of the two equivalent forms to run for n_q new query rows
 * per sequence ("Decoupled RoPE · MLA Part 2", §5 closing remark: the absorbed form is the decode
 * form, the explicit one pays off when many query rows share each rebuilt key and value; "从零理解
 * MLA", section "实际配置"). Returns 1 when mla_prefill_explicit covers the shape and n_q is at
 * least the row count from which it measured faster than mla_absorb_q + mla_decode_attn +
 * mla_out_proj on this library's kernels (256 new rows per sequence); 0 otherwise, including for
 * invalid arguments. Host-only: launches nothing.
 */
int32_t mla_prefill_prefers_explicit(const mla_config* cfg, int32_t batch, int32_t n_q, int32_t max_seq_len);

/*
 * mla_decode_advance — cache growth between decode steps ("从零理解 MLA", the token-by-token
 * decode loop of its decoupled-RoPE check: every step appends the new token and the next one
 * attends to one more key). On the device, enqueued on `stream`:
 *   len_before[b] += n_new and seq_len[b] += n_new for b < batch;  q_pos[r] += n_new for r < n_rows.
 * Any of the three arrays may be NULL (left alone). With the other calls enqueued on the same
 * stream, one recorded step (a captured HIP graph) can be replayed for the next token.
 */
mla_status mla_decode_advance(int32_t batch, int32_t n_new, int32_t* len_before, int32_t* seq_len,
                              int32_t n_rows, int32_t* q_pos, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
