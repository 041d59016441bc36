// Query absorption and latent output projection for the DeepSeek-V2/V3 shape
// (128 heads, d_nope = d_v = 128, d_latent = 512, d_rope = 64, bf16 weights).
//
// At decode batch sizes both calls are matrix-vector products whose cost is reading the
// per-head weights once (W_UK and W_UV are 16.8 MB each in bf16), so the kernels are built for
// HBM streaming: every lane issues independent 16-byte weight loads, a workgroup owns one 32 KB
// weight slab, and 512 workgroups (two per CU) cover the weights once. Query rows are processed
// kRowBlock at a time against the same weight registers.
//
//   absorb: q~[r, i, c] = sum_a W_UK[i, a, c] q_nope[r, i, a]   ("从零理解 MLA", section "矩阵吸收")
//   out:    o[r, i, v]  = sum_c W_UV[i, v, c] z[r, i, c]        (same section, output side)
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace proj {

constexpr int H = 128;
constexpr int DN = 128;   // d_nope = d_v
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;
constexpr int kRowBlock = 4;

__device__ __forceinline__ void unpack8(const i32x4 v, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = (uint32_t)v[e];
    f[2 * e] = __uint_as_float(u << 16);
    f[2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
}

// grid (H, 4 column quarters, row blocks of RB): 512 workgroups of 256 threads, two per CU, each
// streaming a 32 KB slab of W_UK[i] (128 rows x 128 columns) with 8 independent 16-byte loads per
// lane. Column group cg = t % 16 (8 columns), row group ag = t / 16 (8 rows a). The partial sums
// of the 4 row groups of a wave meet by lane exchanges, those of the 4 waves in LDS. The first
// quarter also rotates the rows' position queries while the weights are in flight.
// In a decode step (ap.cache set) the grid has one more column of workgroups, x = H: workgroup
// (H, y, z) appends the new token of row z RB + y (y < RB), and the query positions come from
// ap.seq_len; the append costs no launch of its own.
template <int RB>
__global__ void __launch_bounds__(256) absorb_q_gemv(const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
                                                     const int32_t* __restrict__ q_pos, const bf16* __restrict__ w_uk,
                                                     bf16* __restrict__ q_packed, int n_rows, double base,
                                                     StepAppend ap) {
  __shared__ float qs[RB][DN];
  __shared__ f32x4 red[4][RB][32];   // [wave][row][column quad]
  const int i = blockIdx.x, quarter = blockIdx.y;
  const int r0 = blockIdx.z * RB;
  const int nr = min(RB, n_rows - r0);
  const int t = threadIdx.x, cg = t & 15, ag = t >> 4, w = t >> 6;
  if (i == H) {   // the step's cache append (the whole workgroup takes this branch)
    const int r = r0 + quarter;
    if (quarter >= RB || r >= n_rows) return;
    const int b = r / ap.n_q;
    const int64_t p = (int64_t)ap.seq_len[b] - ap.n_q + r % ap.n_q;
    append_token<bf16>((const bf16*)ap.c_new + (size_t)r * DC, (const bf16*)ap.k_new + (size_t)r * DR,
                       (bf16*)ap.cache + (ap.seq_off[b] + p) * (int64_t)ROW, p, DC, DR, base, ap.vec != 0, t, 256);
    return;
  }
  // weights first: 8 independent 16-byte loads per lane
  const bf16* wp = w_uk + ((size_t)i * DN + ag * 8) * DC + quarter * 128 + cg * 8;
  i32x4 wv[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) wv[a] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp + (size_t)a * DC));
  // while they are in flight: rotate the position part of these rows
  if (quarter == 0) {
    for (int e = t; e < nr * (DR / 2); e += 256) {
      const int rr = e / (DR / 2), j = e % (DR / 2);
      const size_t r = (size_t)(r0 + rr);
      const bf16* src = q_rope + (r * H + i) * DR;
      float sn, co;
      const int pos = q_pos != nullptr ? q_pos[r] : ap.seq_len[r / ap.n_q] - ap.n_q + (int)(r % ap.n_q);
      rope_sincos(rope_theta(base, j, DR), pos, &sn, &co);
      const float x0 = (float)src[2 * j], x1 = (float)src[2 * j + 1];
      bf16* dst = q_packed + (r * H + i) * ROW + DC;
      dst[2 * j] = (bf16)(x0 * co - x1 * sn);
      dst[2 * j + 1] = (bf16)(x0 * sn + x1 * co);
    }
  }
  for (int e = t; e < RB * DN; e += 256) {
    const int rr = e / DN, a = e % DN;
    qs[rr][a] = rr < nr ? (float)q_nope[((size_t)(r0 + rr) * H + i) * DN + a] : 0.0f;
  }
  __syncthreads();
  float acc[RB][8];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[rr][e] = 0.0f;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    float wf[8];
    unpack8(wv[a], wf);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float q = qs[rr][ag * 8 + a];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rr][e] = fmaf(wf[e], q, acc[rr][e]);
    }
  }
  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same 8 columns for the wave's 4 row groups
#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[rr][e] += __shfl_xor(acc[rr][e], 16, 64);
      acc[rr][e] += __shfl_xor(acc[rr][e], 32, 64);
    }
  if ((t & 63) < 16)
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      red[w][rr][2 * cg] = f32x4{acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]};
      red[w][rr][2 * cg + 1] = f32x4{acc[rr][4], acc[rr][5], acc[rr][6], acc[rr][7]};
    }
  __syncthreads();
  // thread t < 128 sums column t of the quarter over the 4 waves for each row
  if (t < 128)
    for (int rr = 0; rr < nr; ++rr) {
      const float* rp = reinterpret_cast<const float*>(&red[0][rr][0]) + t;
      const float sum = rp[0] + rp[RB * 128] + rp[2 * RB * 128] + rp[3 * RB * 128];
      q_packed[((size_t)(r0 + rr) * H + i) * ROW + quarter * 128 + t] = (bf16)sum;
    }
}

// grid (H, 4 quarters of the 128 outputs, row blocks); 4 waves, wave w owns 8 outputs
// v = 32 q + 8 w + j. Lane l holds latent columns 8l..8l+7, so one 16-byte load per lane covers a
// whole 512-wide weight row; the 8 per-lane dot products are then reduced across the wave by
// a reduce-scatter butterfly (each halving step keeps half the outputs), 10 exchanges per row.
__global__ void __launch_bounds__(256) out_proj_gemv(const float* __restrict__ z, const bf16* __restrict__ w_uv,
                                                     bf16* __restrict__ o, int n_rows) {
  const int i = blockIdx.x, quarter = blockIdx.y;
  const int r0 = blockIdx.z * kRowBlock;
  const int nr = min(kRowBlock, n_rows - r0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int v0 = quarter * 32 + w * 8;

  i32x4 wv[8];
  const bf16* wp = w_uv + ((size_t)i * DN + v0) * DC + lane * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) wv[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp + (size_t)j * DC));

  for (int rr = 0; rr < nr; ++rr) {
    const float* zp = z + ((size_t)(r0 + rr) * H + i) * DC + lane * 8;
    const f32x4 za = *reinterpret_cast<const f32x4*>(zp);
    const f32x4 zb = *reinterpret_cast<const f32x4*>(zp + 4);
    float d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float wf[8];
      unpack8(wv[j], wf);
      float s = wf[0] * za[0];
      s = fmaf(wf[1], za[1], s);
      s = fmaf(wf[2], za[2], s);
      s = fmaf(wf[3], za[3], s);
      s = fmaf(wf[4], zb[0], s);
      s = fmaf(wf[5], zb[1], s);
      s = fmaf(wf[6], zb[2], s);
      s = fmaf(wf[7], zb[3], s);
      d[j] = s;
    }
    // reduce-scatter: after exchanging with lane ^ 32 keep outputs 0-3 (low half) or 4-7 (high
    // half), then ^16 keeps 2, ^8 keeps 1; lanes with equal bits 5..3 now hold one output each.
    {
      const bool hi = lane & 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float send = hi ? d[j] : d[j + 4];
        const float recv = __shfl_xor(send, 32, 64);
        d[j] = (hi ? d[j + 4] : d[j]) + recv;
      }
    }
    {
      const bool hi = lane & 16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float send = hi ? d[j] : d[j + 2];
        const float recv = __shfl_xor(send, 16, 64);
        d[j] = (hi ? d[j + 2] : d[j]) + recv;
      }
    }
    float s;
    {
      const bool hi = lane & 8;
      const float send = hi ? d[0] : d[1];
      s = (hi ? d[1] : d[0]) + __shfl_xor(send, 8, 64);
    }
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 1, 64);
    // lane bits: b5 -> output bit 2, b4 -> bit 1, b3 -> bit 0
    const int j = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
    if ((lane & 7) == 0) o[((size_t)(r0 + rr) * H + i) * DN + v0 + j] = (bf16)s;
  }
}

}  // namespace proj

bool proj_fast_supported(const LayerDims& L) {
  return L.n_heads == proj::H && L.d_nope == proj::DN && L.d_v == proj::DN && L.d_latent == proj::DC &&
         L.d_rope == proj::DR;
}

hipError_t launch_absorb_q_fast(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream,
                                const StepAppend* ap) {
  const StepAppend none{nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0};
  const int gx = proj::H + (ap != nullptr ? 1 : 0);
  if (n_rows == 1) {
    hipLaunchKernelGGL(proj::absorb_q_gemv<1>, dim3(gx, 4, 1), dim3(256), 0, stream, (const bf16*)q_nope,
                       (const bf16*)q_rope, q_pos, (const bf16*)w_uk, (bf16*)q_packed, n_rows, L.rope_base,
                       ap != nullptr ? *ap : none);
  } else {
    const int rb = (n_rows + proj::kRowBlock - 1) / proj::kRowBlock;
    hipLaunchKernelGGL(proj::absorb_q_gemv<proj::kRowBlock>, dim3(gx, 4, rb), dim3(256), 0, stream,
                       (const bf16*)q_nope, (const bf16*)q_rope, q_pos, (const bf16*)w_uk, (bf16*)q_packed, n_rows,
                       L.rope_base, ap != nullptr ? *ap : none);
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_fast(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                hipStream_t stream) {
  const int rb = (n_rows + proj::kRowBlock - 1) / proj::kRowBlock;
  hipLaunchKernelGGL(proj::out_proj_gemv, dim3(proj::H, 4, rb), dim3(256), 0, stream, z, (const bf16*)w_uv, (bf16*)o,
                     n_rows);
  return hipGetLastError();
}

}  // namespace mla
