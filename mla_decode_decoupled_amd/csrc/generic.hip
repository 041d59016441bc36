// Shape-generic kernels (VALU, float32 accumulation) for every call of the library.
// They cover any small configuration (the fp32 tiny workload, the hand-worked example, odd
// head counts) and are the fallback for bf16 shapes without a specialised MFMA kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {

// ------------------------------------------------------------------------------ append
// One block per new token, which stores the token's cache row with append_token ("Decoupled
// RoPE · MLA Part 2", §3.4 and §4.3).
template <typename T>
__global__ void __launch_bounds__(128) rope_append_kernel(const T* __restrict__ c_new, const T* __restrict__ k_new,
                                                          T* __restrict__ cache, const int64_t* __restrict__ seq_off,
                                                          const int32_t* __restrict__ len_before, int n_new,
                                                          int d_latent, int d_rope, double base, int vec) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t p = (int64_t)len_before[b] + i;
  const size_t tok = (size_t)b * n_new + i;
  append_token<T>(c_new + tok * d_latent, k_new + tok * d_rope, cache + (seq_off[b] + p) * (int64_t)(d_latent + d_rope),
                  p, d_latent, d_rope, base, vec != 0, threadIdx.x, blockDim.x);
}

// ----------------------------------------------------------------------------- absorb
// q_packed[r, i, c] = sum_a W_UK[i, a, c] q_nope[r, i, a]; a block owns one head, 256 latent
// columns and kAbsRows query rows so each weight element is read once per row tile.
constexpr int kAbsRows = 8;
constexpr int kMaxNope = 256;

template <typename T>
__global__ void __launch_bounds__(256) absorb_q_generic(const T* __restrict__ q_nope, const T* __restrict__ q_rope,
                                                        const int32_t* __restrict__ q_pos, const T* __restrict__ w_uk,
                                                        T* __restrict__ q_packed, int n_rows, int H, int d_nope,
                                                        int d_latent, int d_rope, double base) {
  __shared__ float qs[kAbsRows][kMaxNope];
  const int i = blockIdx.y;
  const int r0 = blockIdx.x * kAbsRows;
  const int nr = min(kAbsRows, n_rows - r0);
  const int row = d_latent + d_rope;
  for (int e = threadIdx.x; e < kAbsRows * d_nope; e += blockDim.x) {
    const int rr = e / d_nope, a = e % d_nope;
    qs[rr][a] = rr < nr ? to_f32(q_nope[((size_t)(r0 + rr) * H + i) * d_nope + a]) : 0.0f;
  }
  __syncthreads();
  const int c = blockIdx.z * blockDim.x + threadIdx.x;
  if (c < d_latent) {
    float acc[kAbsRows];
#pragma unroll
    for (int rr = 0; rr < kAbsRows; ++rr) acc[rr] = 0.0f;
    const T* w = w_uk + (size_t)i * d_nope * d_latent + c;
    for (int a = 0; a < d_nope; ++a) {
      const float wv = to_f32(w[(size_t)a * d_latent]);
#pragma unroll
      for (int rr = 0; rr < kAbsRows; ++rr) acc[rr] = fmaf(wv, qs[rr][a], acc[rr]);
    }
    for (int rr = 0; rr < nr; ++rr) q_packed[((size_t)(r0 + rr) * H + i) * row + c] = from_f32<T>(acc[rr]);
  }
  if (blockIdx.z == 0) {
    const int half = d_rope / 2;
    for (int e = threadIdx.x; e < nr * half; e += blockDim.x) {
      const int rr = e / half, j = e % half;
      const size_t r = (size_t)(r0 + rr);
      const T* src = q_rope + (r * H + i) * d_rope;
      double s, co;
      rope_sincos_f64(rope_theta(base, j, d_rope), q_pos[r], &s, &co);
      const double x0 = to_f32(src[2 * j]), x1 = to_f32(src[2 * j + 1]);
      T* dst = q_packed + (r * H + i) * row + d_latent;
      dst[2 * j] = from_f64<T>(x0 * co - x1 * s);
      dst[2 * j + 1] = from_f64<T>(x0 * s + x1 * co);
    }
  }
}

// ------------------------------------------------------------------------ attention
// One block per (split chunk, query row, head). Keys of the chunk are taken 256 at a time:
// each thread scores one key over the whole packed row, the block keeps an online softmax
// (running max in log2 units, running sum) and every thread accumulates a few latent columns.
constexpr int kGenMaxRow = 1024;
constexpr int kGenCols = kGenMaxRow / 256;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  v = is_max ? warp_max(v) : warp_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  const int nw = blockDim.x >> 6;
  for (int k = 1; k < nw; ++k) r = is_max ? fmaxf(r, red[k]) : r + red[k];
  return r;
}

template <typename T>
__global__ void __launch_bounds__(256) attn_partial_generic(const T* __restrict__ q_packed, const T* __restrict__ cache,
                                                            const int64_t* __restrict__ seq_off,
                                                            const int32_t* __restrict__ seq_len, int n_q, int H,
                                                            int d_latent, int d_rope, float scale_log2, int chunk_len,
                                                            int n_chunks, float* __restrict__ part_acc,
                                                            float* __restrict__ part_ml, float* __restrict__ z,
                                                            float* __restrict__ lse) {
  __shared__ float qs[kGenMaxRow];
  __shared__ float ps[256];
  __shared__ float red[8];
  const int k = blockIdx.x, bt = blockIdx.y, i = blockIdx.z;
  const int b = bt / n_q, t = bt % n_q;
  const int row = d_latent + d_rope;
  const int n_vis = seq_len[b] - n_q + t + 1;
  const int j0 = k * chunk_len;
  const int j1 = min(j0 + chunk_len, n_vis);
  const T* q = q_packed + ((size_t)bt * H + i) * row;
  for (int d = threadIdx.x; d < row; d += blockDim.x) qs[d] = to_f32(q[d]);
  __syncthreads();
  const T* kv = cache + seq_off[b] * (int64_t)row;

  float m = -INFINITY, l = 0.0f;
  float acc[kGenCols];
#pragma unroll
  for (int u = 0; u < kGenCols; ++u) acc[u] = 0.0f;

  for (int jt = j0; jt < j1; jt += blockDim.x) {
    const int j = jt + threadIdx.x;
    float s = -INFINITY;
    if (j < j1) {
      const T* kr = kv + (int64_t)j * row;
      float dot = 0.0f;
      for (int d = 0; d < row; ++d) dot = fmaf(qs[d], to_f32(kr[d]), dot);
      s = dot * scale_log2;
    }
    const float m_new = fmaxf(m, block_reduce(s, true, red));
    const float alpha = exp2f(m - m_new);
    const float p = (j < j1) ? exp2f(s - m_new) : 0.0f;
    ps[threadIdx.x] = p;
    l = l * alpha + block_reduce(p, false, red);
    __syncthreads();
    const int nt = min((int)blockDim.x, j1 - jt);
#pragma unroll
    for (int u = 0; u < kGenCols; ++u) {
      const int c = threadIdx.x + u * blockDim.x;
      if (c < d_latent) {
        float a = acc[u] * alpha;
        const T* col = kv + (int64_t)jt * row + c;
        for (int jj = 0; jj < nt; ++jj) a = fmaf(ps[jj], to_f32(col[(int64_t)jj * row]), a);
        acc[u] = a;
      }
    }
    m = m_new;
    __syncthreads();
  }

  const size_t rh = (size_t)bt * H + i;
  if (n_chunks == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int u = 0; u < kGenCols; ++u) {
      const int c = threadIdx.x + u * blockDim.x;
      if (c < d_latent) z[rh * d_latent + c] = acc[u] * inv;
    }
    if (lse != nullptr && threadIdx.x == 0) lse[rh] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
  } else {
    const size_t slot = rh * n_chunks + k;
#pragma unroll
    for (int u = 0; u < kGenCols; ++u) {
      const int c = threadIdx.x + u * blockDim.x;
      if (c < d_latent) part_acc[slot * d_latent + c] = acc[u];
    }
    if (threadIdx.x == 0) {
      part_ml[slot * 2 + 0] = m;
      part_ml[slot * 2 + 1] = l;
    }
  }
}

// Log-sum-exp merge of split-K partials of one (query row, head): with M = max_k m_k,
// z = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k. Chunks that saw no key (l_k = 0) are
// skipped (their accumulator is never read), so an empty chunk never produces NaN.
//
// The merge is a pure stream over the partials, so it is written for memory-level parallelism:
// wave 0 first compacts the live chunks and their weights into LDS, then the 4 waves split the
// live chunks round-robin, every lane reading V consecutive floats of each chunk row with all of a
// batch of 8 chunk loads in flight before the first is used; the 4 wave sums meet in LDS.
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 8;

template <int V>
__global__ void __launch_bounds__(256) attn_merge(const float* __restrict__ part_acc, const float* __restrict__ part_ml,
                                                  int n_chunks, int d_latent, float* __restrict__ z,
                                                  float* __restrict__ lse) {
  typedef __attribute__((__vector_size__(V * sizeof(float)))) float vec;
  extern __shared__ __attribute__((aligned(16))) float merge_smem[];
  float* red = merge_smem;                                       // [kMergeWaves][d_latent]
  float* wts = red + kMergeWaves * d_latent;                     // [kMaxSplits] live weights
  int* idx = reinterpret_cast<int*>(wts + kMaxSplits);           // [kMaxSplits] live chunk ids
  __shared__ int n_live;
  __shared__ float total;
  const size_t rh = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w == 0) {
    const float* ml = part_ml + rh * n_chunks * 2;
    float M = -INFINITY;
    for (int k = lane; k < n_chunks; k += 64)
      if (ml[2 * k + 1] > 0.0f) M = fmaxf(M, ml[2 * k]);
    M = warp_max(M);
    float L = 0.0f;
    int base = 0;
    for (int k0 = 0; k0 < n_chunks; k0 += 64) {
      const int k = k0 + lane;
      const float m = k < n_chunks ? ml[2 * k] : 0.0f;
      const float l = k < n_chunks ? ml[2 * k + 1] : 0.0f;
      const bool live = l > 0.0f;
      const uint64_t mask = __ballot(live);
      if (live) {
        const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
        const float wk = exp2f(m - M);
        wts[pos] = wk;
        idx[pos] = k;
        L = fmaf(wk, l, L);
      }
      base += __popcll(mask);
    }
    L = warp_sum(L);
    if (lane == 0) {
      n_live = base;
      total = L;
      if (lse != nullptr) lse[rh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  const int live = n_live;
  const float* acc = part_acc + rh * n_chunks * (size_t)d_latent;
  for (int c = lane * V; c < d_latent; c += 64 * V) {
    vec s = {};
    for (int q0 = w; q0 < live; q0 += kMergeWaves * kMergeBatch) {
      vec x[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int q = q0 + u * kMergeWaves;
        if (q < live) x[u] = *reinterpret_cast<const vec*>(acc + (size_t)idx[q] * d_latent + c);
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int q = q0 + u * kMergeWaves;
        if (q < live) s += wts[q] * x[u];
      }
    }
    *reinterpret_cast<vec*>(red + w * d_latent + c) = s;
  }
  __syncthreads();
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;
  for (int c = threadIdx.x; c < d_latent; c += blockDim.x) {
    float s = 0.0f;
#pragma unroll
    for (int g = 0; g < kMergeWaves; ++g) s += red[g * d_latent + c];
    z[rh * d_latent + c] = s * inv;
  }
}

// ------------------------------------------------------------------------- out proj
// o[r, i, v] = sum_c W_UV[i, v, c] z[r, i, c]: one block per (row tile, head); each wave
// takes output columns v in turn and reduces over the latent with its 64 lanes.
constexpr int kOutRows = 4;

template <typename T>
__global__ void __launch_bounds__(256) out_proj_generic(const float* __restrict__ z, const T* __restrict__ w_uv,
                                                        T* __restrict__ o, int n_rows, int H, int d_latent, int d_v) {
  __shared__ float zs[kOutRows][kGenMaxRow];
  const int i = blockIdx.y;
  const int r0 = blockIdx.x * kOutRows;
  const int nr = min(kOutRows, n_rows - r0);
  for (int e = threadIdx.x; e < kOutRows * d_latent; e += blockDim.x) {
    const int rr = e / d_latent, c = e % d_latent;
    zs[rr][c] = rr < nr ? z[((size_t)(r0 + rr) * H + i) * d_latent + c] : 0.0f;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int v = w; v < d_v; v += blockDim.x >> 6) {
    const T* wr = w_uv + ((size_t)i * d_v + v) * d_latent;
    float acc[kOutRows] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = lane; c < d_latent; c += 64) {
      const float wv = to_f32(wr[c]);
#pragma unroll
      for (int rr = 0; rr < kOutRows; ++rr) acc[rr] = fmaf(wv, zs[rr][c], acc[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < kOutRows; ++rr) acc[rr] = warp_sum(acc[rr]);
    if (lane == 0)
      for (int rr = 0; rr < nr; ++rr) o[((size_t)(r0 + rr) * H + i) * d_v + v] = from_f32<T>(acc[rr]);
  }
}

// -------------------------------------------------------------------------- launchers
bool append_vec_ok(const LayerDims& L, size_t elem_bytes, const void* c_new, const void* cache) {
  return ((size_t)L.d_latent * elem_bytes) % 16 == 0 && ((size_t)(L.d_latent + L.d_rope) * elem_bytes) % 16 == 0 &&
         ((uintptr_t)c_new & 15u) == 0 && ((uintptr_t)cache & 15u) == 0;
}

template <typename T>
hipError_t launch_rope_append_generic(const LayerDims& L, int batch, int n_new, const void* c_new,
                                      const void* k_new, void* cache, const int64_t* seq_off,
                                      const int32_t* len_before, hipStream_t stream) {
  dim3 grid(n_new, batch);
  const bool vec = append_vec_ok(L, sizeof(T), c_new, cache);
  hipLaunchKernelGGL(rope_append_kernel<T>, grid, dim3(128), 0, stream, (const T*)c_new, (const T*)k_new, (T*)cache,
                     seq_off, len_before, n_new, L.d_latent, L.d_rope, L.rope_base, vec ? 1 : 0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_absorb_q_generic(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                   const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream) {
  dim3 grid((n_rows + kAbsRows - 1) / kAbsRows, L.n_heads, (L.d_latent + 255) / 256);
  hipLaunchKernelGGL(absorb_q_generic<T>, grid, dim3(256), 0, stream, (const T*)q_nope, (const T*)q_rope, q_pos,
                     (const T*)w_uk, (T*)q_packed, n_rows, L.n_heads, L.d_nope, L.d_latent, L.d_rope, L.rope_base);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_generic(const LayerDims& L, int batch, int n_q, const void* q_packed, const void* cache,
                               const int64_t* seq_off, const int32_t* seq_len, const SplitPlan& plan,
                               void* workspace, float* z, float* lse, hipStream_t stream) {
  float* part_acc = (float*)workspace;
  float* part_ml = plan.n_chunks > 1 ? part_acc + (size_t)batch * n_q * L.n_heads * plan.n_chunks * L.d_latent : nullptr;
  dim3 grid(plan.n_chunks, batch * n_q, L.n_heads);
  hipLaunchKernelGGL(attn_partial_generic<T>, grid, dim3(256), 0, stream, (const T*)q_packed, (const T*)cache, seq_off,
                     seq_len, n_q, L.n_heads, L.d_latent, L.d_rope, L.softmax_scale * kLog2e, plan.chunk_len,
                     plan.n_chunks, part_acc, part_ml, z, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_chunks == 1) return e;
  return launch_attn_merge(batch * n_q * L.n_heads, plan.n_chunks, L.d_latent, part_acc, part_ml, z, lse, stream);
}

hipError_t launch_attn_merge(int n_rowheads, int n_chunks, int d_latent, const float* part_acc, const float* part_ml,
                             float* z, float* lse, hipStream_t stream) {
  const size_t smem = (size_t)kMergeWaves * d_latent * sizeof(float) + kMaxSplits * (sizeof(float) + sizeof(int));
  if (d_latent % 4 == 0 && ((uintptr_t)part_acc & 15u) == 0)
    hipLaunchKernelGGL(attn_merge<4>, dim3(n_rowheads), dim3(64 * kMergeWaves), smem, stream, part_acc, part_ml,
                       n_chunks, d_latent, z, lse);
  else
    hipLaunchKernelGGL(attn_merge<1>, dim3(n_rowheads), dim3(64 * kMergeWaves), smem, stream, part_acc, part_ml,
                       n_chunks, d_latent, z, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_out_proj_generic(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                   hipStream_t stream) {
  dim3 grid((n_rows + kOutRows - 1) / kOutRows, L.n_heads);
  hipLaunchKernelGGL(out_proj_generic<T>, grid, dim3(256), 0, stream, z, (const T*)w_uv, (T*)o, n_rows, L.n_heads,
                     L.d_latent, L.d_v);
  return hipGetLastError();
}

// ------------------------------------------------------------------- decode advance
// After a decode step that appended n_new tokens to every sequence, the next step's append
// position, key count and query positions each move on by n_new (the cache grows by the tokens
// just written; "从零理解 MLA", decode loop of the decoupled-RoPE check). One thread per entry.
__global__ void __launch_bounds__(256) decode_advance(int batch, int n_new, int32_t* __restrict__ len_before,
                                                      int32_t* __restrict__ seq_len, int n_rows,
                                                      int32_t* __restrict__ q_pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < batch) {
    if (len_before != nullptr) len_before[i] += n_new;
    if (seq_len != nullptr) seq_len[i] += n_new;
  }
  if (i < n_rows && q_pos != nullptr) q_pos[i] += n_new;
}

hipError_t launch_decode_advance(int batch, int n_new, int32_t* len_before, int32_t* seq_len, int n_rows,
                                 int32_t* q_pos, hipStream_t stream) {
  const int n = batch > n_rows ? batch : n_rows;
  hipLaunchKernelGGL(decode_advance, dim3((n + 255) / 256), dim3(256), 0, stream, batch, n_new, len_before, seq_len,
                     n_rows, q_pos);
  return hipGetLastError();
}

// Positions of a decode step's new tokens from the key counts (mla_decode_step): row r = b n_q + t
// of sequence b is the token at position seq_len[b] - n_q + t, and sequence b's first new token
// goes after its seq_len[b] - n_q cached ones. One thread per row.
__global__ void __launch_bounds__(256) step_positions(const int32_t* __restrict__ seq_len, int n_q, int n_rows,
                                                      int32_t* __restrict__ len_before, int32_t* __restrict__ q_pos) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const int b = r / n_q, t = r % n_q;
  const int32_t first = seq_len[b] - n_q;
  q_pos[r] = first + t;
  if (t == 0) len_before[b] = first;
}

hipError_t launch_step_positions(const int32_t* seq_len, int batch, int n_q, int32_t* len_before, int32_t* q_pos,
                                 hipStream_t stream) {
  const int rows = batch * n_q;
  hipLaunchKernelGGL(step_positions, dim3((rows + 255) / 256), dim3(256), 0, stream, seq_len, n_q, rows, len_before,
                     q_pos);
  return hipGetLastError();
}

#define MLA_INSTANTIATE(T)                                                                                        \
  template hipError_t launch_rope_append_generic<T>(const LayerDims&, int, int, const void*, const void*, void*,  \
                                                    const int64_t*, const int32_t*, hipStream_t);                \
  template hipError_t launch_absorb_q_generic<T>(const LayerDims&, int, const void*, const void*, const int32_t*, \
                                                 const void*, void*, hipStream_t);                               \
  template hipError_t launch_attn_generic<T>(const LayerDims&, int, int, const void*, const void*, const int64_t*, \
                                             const int32_t*, const SplitPlan&, void*, float*, float*, hipStream_t); \
  template hipError_t launch_out_proj_generic<T>(const LayerDims&, int, const float*, const void*, void*, hipStream_t);

MLA_INSTANTIATE(float)
MLA_INSTANTIATE(bf16)

}  // namespace mla
