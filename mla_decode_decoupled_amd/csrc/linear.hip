// Upstream projections of one MLA layer: from the hidden state h to the inputs of the cache append
// and of the query absorption.
//   kv side ("Decoupled RoPE · MLA Part 2", §5 steps 2–3; "构建DeepSeek-V3：MLA 架构", step 1):
//     c = RMSNorm(W_DKV h) (the norm is optional), k_R = RoPE_p(W_KR h), stored as the token's
//     packed cache row [c ; k_R];
//   query side ("从零理解 MLA", sections "查询压缩" and "解耦 RoPE"; "构建DeepSeek-V3：MLA 架构",
//     query compression): c_Q = W_DQ h, q_C = W_UQ c_Q, q_R = W_QR c_Q (unrotated; mla_absorb_q
//     rotates it), or q_C = W_Q h, q_R = W_QR h without query compression.
//
// Every product is a linear layer y[r, n] = sum_k x[r, k] W[n, k] with W in nn.Linear's [out, in]
// layout. Two weights that read the same x (W_DKV and W_KR; W_UQ and W_QR) run as one launch over
// their concatenated rows ("segments"), each segment writing its own output. Three kernels:
//   * lin_generic: any shape and dtype, one wave per output column;
//   * lin_gemv (bf16, few rows): weight-bandwidth bound. A wave owns RW weight rows, its lanes
//     stream them with nontemporal 16-byte loads (several per lane in flight) next to the matching
//     pieces of the RB activation rows (read through the caches, where every workgroup finds them);
//   * lin_gemm (bf16, many rows): MFMA 32x32x16, 128 x 128 outputs per workgroup, both operands
//     K-contiguous and staged through padded LDS rows, the next K step's loads in flight during the
//     MFMAs;
//   * lin_gemm_wide (bf16 in and out, 256 rows or more): 256 x 128 outputs per workgroup, operands
//     loaded straight into LDS, two workgroups per CU (also the key/value rebuild of the explicit
//     prefill).
// Accumulation is float32; each output is rounded once to its type.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace lin {

// output columns [0, n1) come from weight w1 and go to y1 (row stride ldy1); [n1, n) from w2 / y2
struct Seg2 {
  const void* w1;
  const void* w2;
  void* y1;
  void* y2;
  int n1, n, ldy1, ldy2;
};

template <typename T>
__device__ __forceinline__ const T* wrow(const Seg2& s, int n, int K) {
  return n < s.n1 ? (const T*)s.w1 + (size_t)n * K : (const T*)s.w2 + (size_t)(n - s.n1) * K;
}
template <typename Ty>
__device__ __forceinline__ void ystore(const Seg2& s, int r, int n, float v) {
  if (n < s.n1)
    ((Ty*)s.y1)[(size_t)r * s.ldy1 + n] = from_f32<Ty>(v);
  else
    ((Ty*)s.y2)[(size_t)r * s.ldy2 + (n - s.n1)] = from_f32<Ty>(v);
}

// Up to three segments for the matrix-vector kernel, each with its own output type: output
// columns [end[k-1], end[k]) come from weight w[k] and go to y[k] (row stride ldy[k]), stored as
// float32 when f32[k] is set, else as bf16.
struct Seg3 {
  const void* w[3];
  void* y[3];
  int end[3];
  int ldy[3];
  int f32[3];
};

__device__ __forceinline__ int seg_of(const Seg3& s, int n) { return n < s.end[0] ? 0 : (n < s.end[1] ? 1 : 2); }
__device__ __forceinline__ int seg_base(const Seg3& s, int k) { return k == 0 ? 0 : s.end[k - 1]; }

// The kv side's finish, carried by a projection launch: RMS-normalise the latent part of a token's
// float32 projection (gain optional), rotate its position part by the token's position in float64,
// and store the packed row into the token's cache slot. pre [rows, d_latent + d_rope] float32; row
// r = b n_new + i is token i of sequence b, at position len_before[b] + i.
struct KvFinish {
  const float* pre;
  const void* norm_w;
  void* cache;
  const int64_t* seq_off;
  const int32_t* len_before;
  float eps;
  int use_norm, n_new, d_latent, d_rope;
  double base;
};

// one token, the whole block (blockDim.x = 256) taking part; red: 4 floats of shared memory
template <typename T>
__device__ void finish_token(const KvFinish& f, int r, float* red) {
  const int row = f.d_latent + f.d_rope;
  const int b = r / f.n_new, i = r % f.n_new;
  const float* src = f.pre + (size_t)r * row;
  const int64_t p = (int64_t)f.len_before[b] + i;
  T* dst = (T*)f.cache + (f.seq_off[b] + p) * (int64_t)row;
  float inv = 1.0f;
  if (f.use_norm) {
    float ss = 0.0f;
    for (int c = threadIdx.x; c < f.d_latent; c += blockDim.x) ss = fmaf(src[c], src[c], ss);
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    __syncthreads();   // red is free for the next token
    inv = 1.0f / sqrtf(tot / (float)f.d_latent + f.eps);
  }
  for (int c = threadIdx.x; c < f.d_latent; c += blockDim.x) {
    float v = src[c] * inv;
    if (f.use_norm && f.norm_w != nullptr) v *= to_f32(((const T*)f.norm_w)[c]);
    dst[c] = from_f32<T>(v);
  }
  for (int j = threadIdx.x; j < f.d_rope / 2; j += blockDim.x) {
    double sn, cs;
    rope_sincos_f64(rope_theta(f.base, j, f.d_rope), p, &sn, &cs);
    const double x0 = src[f.d_latent + 2 * j], x1 = src[f.d_latent + 2 * j + 1];
    dst[f.d_latent + 2 * j] = from_f64<T>(x0 * cs - x1 * sn);
    dst[f.d_latent + 2 * j + 1] = from_f64<T>(x0 * sn + x1 * cs);
  }
}

// ---------------------------------------------------------------- generic
// grid (ceil(n / 4), min(M, 65535)), 256 threads: wave w computes column 4 blockIdx.x + w for rows
// blockIdx.y, blockIdx.y + gridDim.y, ...
template <typename T, typename Ty>
__global__ void __launch_bounds__(256) lin_generic(const T* __restrict__ x, int ldx, int M, int K, Seg2 s) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + w;
  if (n >= s.n) return;
  const T* wr = wrow<T>(s, n, K);
  for (int r = blockIdx.y; r < M; r += gridDim.y) {
    const T* xr = x + (size_t)r * ldx;
    float acc = 0.0f;
    for (int k = lane; k < K; k += 64) acc = fmaf(to_f32(wr[k]), to_f32(xr[k]), acc);
    acc = warp_sum(acc);
    if (lane == 0) ystore<Ty>(s, r, n, acc);
  }
}

__device__ __forceinline__ void unpack8(const i32x4 v, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = (uint32_t)v[e];
    f[2 * e] = __uint_as_float(u << 16);
    f[2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------- few rows
// grid (ceil(n / (RW 4 / KS)) [+ 1 finish column], ceil(M / RB)), 256 threads. The 4 waves form
// 4 / KS groups of KS waves; group g owns weight rows (blockIdx.x (4 / KS) + g) RW .. +RW-1 and the
// KS waves of a group split K between them (wave part p takes the 16-byte pieces
// 64 p + lane + 64 KS j), so a short K still gives every lane several independent loads. Each lane
// keeps RW x U weight loads in flight (nontemporal: the weights are read once) next to the
// matching pieces of the RB activation rows (through the caches, where every workgroup finds
// them). With FIN the first column of workgroups runs finish_token for the rows of its row block
// instead (first, so that it is dispatched at once: the grid can hold more workgroups than the
// chip, and a last column would wait for the others). FIN is a template flag because the float64
// rotation costs registers, and with them occupancy, wherever it is compiled in; with one
// activation row the FIN kernel is held to 7 waves per SIMD (72 VGPRs, the matrix-vector loop's
// own need), so the finish path spills a few registers to scratch in its one workgroup column
// instead of the whole launch running at 4 waves per SIMD (W_UQ + W_QR of the DeepSeek-V3 shape:
// 15.6 us at 7 waves, 16.0 at 6, 17.6 at 4). K % 8 == 0, x and W 16-byte aligned, ldx % 8 == 0.
template <int RW, int RB, int KS, bool FIN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FIN && RB == 1 ? 7 : 1)))
lin_gemv(const bf16* __restrict__ x, int ldx, int M, int K, Seg3 s, KvFinish f) {
  constexpr int U = 8 / RW;
  constexpr int G = 4 / KS;
  __shared__ float red[4][RW][RB];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = w / KS, part = w % KS;
  const int r0 = blockIdx.y * RB, nr = min(RB, M - r0);
  int bx = blockIdx.x;
  if constexpr (FIN) {
    if (bx == 0) {   // the whole workgroup
      for (int rr = 0; rr < nr; ++rr) finish_token<bf16>(f, r0 + rr, &red[0][0][0]);
      return;
    }
    --bx;
  }
  const int n = s.end[2];
  const int nb = (bx * G + grp) * RW;
  const bool active = nb < n;
  const int KP = K / 8;
  const bf16* wr[RW];
  bool ok[RW];
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    ok[q] = nb + q < n;
    const int row = ok[q] ? nb + q : (active ? nb : 0);
    const int k = seg_of(s, row);
    wr[q] = (const bf16*)s.w[k] + (size_t)(row - seg_base(s, k)) * K;
  }
  const bf16* xr[RB];
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) xr[rr] = x + (size_t)(r0 + (rr < nr ? rr : 0)) * ldx;
  float acc[RW][RB];
#pragma unroll
  for (int q = 0; q < RW; ++q)
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) acc[q][rr] = 0.0f;
  if (active) {
#pragma unroll 1
    for (int p0 = 64 * part; p0 < KP; p0 += 64 * KS * U) {
      i32x4 wv[RW][U], xv[RB][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + 64 * KS * u + lane;
        const bool in = p < KP;
#pragma unroll
        for (int q = 0; q < RW; ++q)
          wv[q][u] = in && ok[q] ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wr[q] + 8 * p))
                                 : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
          xv[rr][u] = in && rr < nr ? *reinterpret_cast<const i32x4*>(xr[rr] + 8 * p) : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float xf[RB][8];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) unpack8(xv[rr][u], xf[rr]);
#pragma unroll
        for (int q = 0; q < RW; ++q) {
          float wf[8];
          unpack8(wv[q][u], wf);
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][rr] = fmaf(wf[e], xf[rr][e], acc[q][rr]);
        }
      }
    }
  }
  auto store = [&](int r, int col, float v) {
    const int k = seg_of(s, col);
    const size_t o = (size_t)r * s.ldy[k] + (col - seg_base(s, k));
    if (s.f32[k])
      ((float*)s.y[k])[o] = v;
    else
      ((bf16*)s.y[k])[o] = (bf16)v;
  };
#pragma unroll
  for (int q = 0; q < RW; ++q)
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float v = warp_sum(acc[q][rr]);
      if constexpr (KS == 1) {
        if (lane == 0 && ok[q] && active && rr < nr) store(r0 + rr, nb + q, v);
      } else {
        if (lane == 0) red[w][q][rr] = v;
      }
    }
  if constexpr (KS > 1) {
    __syncthreads();
    if (part == 0 && lane == 0 && active) {
#pragma unroll
      for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          float v = red[w][q][rr];
#pragma unroll
          for (int k = 1; k < KS; ++k) v += red[w + k][q][rr];
          if (ok[q] && rr < nr) store(r0 + rr, nb + q, v);
        }
    }
  }
}

// ---------------------------------------------------------------- many rows
typedef __bf16 bf16x8e __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int SROW = TK + 8;   // bf16 per staged row (80 bytes: 16 lanes of a 16-byte read hit 16 bank groups)
constexpr int GEMM_LDS = 2 * 2 * TM * SROW * 2;   // two buffers of the A and B tiles

// Per-sequence rows (SEQ form): blockIdx.z is a sequence b whose M = len[b] rows start at row
// off[b] of x; its outputs start y_bstride elements further per b. The row tile is blockIdx.x
// and the column tile blockIdx.y in this form. With head_stride > 0 (lin_gemm_wide only) a
// segment's outputs are stored head-major instead: its columns in blocks of 128, block h of row m
// at h * head_stride + 128 m, so that one head's rows are contiguous.
struct SeqRows {
  const int32_t* len;
  const int64_t* off;
  int64_t y_bstride;
  int64_t head_stride = 0;
};

// grid (ceil(n / 128), ceil(M / 128)), or (ceil(M / 128), ceil(n / 128), sequences) in the SEQ form;
// 256 threads, GEMM_LDS dynamic LDS; K % 32 == 0.
// Wave w computes rows 64 (w / 2) .. +63 and columns 64 (w % 2) .. +63 of the tile: 2 x 2 MFMA
// blocks of 32 x 32. Per K step of 32, every thread moves 2 x 16 bytes of A (x rows) and of B
// (weight rows) global -> registers -> LDS; the next step's loads are in flight during the MFMAs.
// STAGED (bf16 outputs whose rows and segments allow 16-byte stores): the MFMAs compute the tile
// transposed, D[n][m], so each lane holds 4 consecutive outputs of one row; the tile is staged in
// LDS and written back with 16-byte stores, 16 lanes per 256-byte row.
constexpr int CS_STRIDE = TN + 8;   // bf16 per staged output row (272 bytes)
static_assert(TM * CS_STRIDE * 2 <= GEMM_LDS, "output staging fits the operand buffers");

template <typename Ty, bool SEQ, bool STAGED>
__global__ void __launch_bounds__(256) lin_gemm(const bf16* __restrict__ x, int ldx, int M, int K, Seg2 s,
                                                SeqRows sq) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if constexpr (SEQ) {
    const int b = blockIdx.z;
    M = sq.len[b];
    if ((int)blockIdx.x * TM >= M) return;   // whole workgroup, before any barrier
    x += sq.off[b] * (int64_t)ldx;
    s.y1 = (Ty*)s.y1 + b * sq.y_bstride;
    s.y2 = (Ty*)s.y2 + b * sq.y_bstride;
  }
  bf16* As = reinterpret_cast<bf16*>(smem);   // [2][TM][SROW]
  bf16* Bs = As + 2 * TM * SROW;              // [2][TN][SROW]
  // SEQ grids run the row tiles fastest: the workgroups dealt to one XCD then share a weight tile
  // and a few row tiles through its L2 (the per-sequence products have a short K)
  const int m0 = (SEQ ? blockIdx.x : blockIdx.y) * TM, n0 = (SEQ ? blockIdx.y : blockIdx.x) * TN;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // loader: thread t moves rows t / 4 and 64 + t / 4, 16-byte piece t % 4 of each K step
  const int lr = t >> 2, lc = (t & 3) * 8;
  const bf16* ga[2];
  const bf16* gb[2];
  bool va[2], vb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ra = m0 + lr + 64 * h, rb = n0 + lr + 64 * h;
    va[h] = ra < M;
    vb[h] = rb < s.n;
    ga[h] = x + (size_t)(va[h] ? ra : 0) * ldx + lc;
    gb[h] = wrow<bf16>(s, vb[h] ? rb : 0, K) + lc;
  }
  i32x4 ra_[2], rb_[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra_[h] = va[h] ? *reinterpret_cast<const i32x4*>(ga[h] + k0) : i32x4{0, 0, 0, 0};
      rb_[h] = vb[h] ? *reinterpret_cast<const i32x4*>(gb[h] + k0) : i32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<i32x4*>(As + ((size_t)buf * TM + lr + 64 * h) * SROW + lc) = ra_[h];
      *reinterpret_cast<i32x4*>(Bs + ((size_t)buf * TN + lr + 64 * h) * SROW + lc) = rb_[h];
    }
  };
  f32x16e acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16e{};
  const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
  gload(0);
  lstore(0);
  __syncthreads();
  const int NK = K / TK;
  for (int kt = 0; kt < NK; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < NK) gload((kt + 1) * TK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8e af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8e*>(As + ((size_t)buf * TM + wm + 32 * i + l32) * SROW + 16 * ks + 8 * g);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8e*>(Bs + ((size_t)buf * TN + wn + 32 * j + l32) * SROW + 16 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = STAGED ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < NK) {
      lstore(buf ^ 1);   // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  if constexpr (STAGED) {
    // D^T block (i, j): lane holds row m = l32 of block i, columns 8 q + 4 g + e of block j
    __syncthreads();   // every wave is done with the operand buffers
    bf16* Cs = As;     // [TM][CS_STRIDE]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][4 * q + e];
          *reinterpret_cast<bf16x4*>(Cs + (wm + 32 * i + l32) * CS_STRIDE + wn + 32 * j + 8 * q + 4 * g) = v;
        }
    __syncthreads();
    const int c = t & 15;
#pragma unroll
    for (int k = 0; k < TM / 16; ++k) {
      const int r = (t >> 4) + 16 * k;
      const int m = m0 + r, n = n0 + 8 * c;
      if (m < M && n < s.n) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(Cs + r * CS_STRIDE + 8 * c);
        bf16* dst = n < s.n1 ? (bf16*)s.y1 + (size_t)m * s.ldy1 + n : (bf16*)s.y2 + (size_t)m * s.ldy2 + (n - s.n1);
        *reinterpret_cast<i32x4*>(dst) = v;
      }
    }
    return;
  }
  // D block (i, j): lane holds column n = l32, rows 8 q + 4 g + e (register 4 q + e)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      if (n >= s.n) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm + 32 * i + 8 * q + 4 * g + e;
          if (m < M) ystore<Ty>(s, m, n, acc[i][j][4 * q + e]);
        }
    }
}

// ---------------------------------------------------------------- many rows, wide tiles
// 256 x 128 outputs per workgroup for large GEMMs (the key/value rebuild of the explicit prefill),
// two workgroups per CU so that one's loads, barriers and output stores overlap the other's
// MFMAs: each of the 4 waves owns 128 x 64 outputs (4 x 2 MFMA blocks, 128 accumulators). K steps
// of 32: both operand tiles (rows x 64 B) reach LDS by direct 1 KB global->LDS loads (no staging
// registers) into a ring of three stages, two steps' loads in flight during a step's MFMAs;
// 16-byte piece c of LDS row r sits at slot c ^ ((r >> 2) & 3), so the 16 rows read together by
// a fragment load fall on distinct bank groups. Outputs are computed transposed, D[n][m], staged
// in LDS and written with 16-byte stores (bf16 outputs whose rows and segments allow them).
// grid (ceil(n / 128), ceil(M / 256)), or (ceil(M / 256), ceil(n / 128), sequences) in the SEQ
// form; 256 threads, WIDE_LDS dynamic LDS; K % 32 == 0, x and weights 16-byte aligned, ldx % 8 == 0.
constexpr int WM = 256, WN = 128, WK = 32, WSTAGES = 3;
constexpr int WROW = WK * 2;                         // 64 bytes per staged operand row
constexpr int WBUF = (WM + WN) * WROW;               // A and B of one K step (24 KB)
constexpr int WLOADS = (WM + WN) / 64;               // 1 KB loads per wave and K step
constexpr int WCS = WN + 8;                          // bf16 per staged output row (272 bytes)
constexpr int WIDE_LDS = WM * WCS * 2 > WSTAGES * WBUF ? WM * WCS * 2 : WSTAGES * WBUF;
static_assert(2 * WIDE_LDS <= 160 * 1024, "two workgroups per CU");

__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ int wslot(int c, int r) { return c ^ ((r >> 2) & 3); }
// Barrier for LDS traffic only: __syncthreads() would also wait for the loads in flight (its
// fence covers the global->LDS loads), which would empty the ring at every step.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// wait until at most N of this wave's loads are in flight; vmcnt: bits 3:0 and 15:14
template <int N>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool SEQ>
__global__ void __launch_bounds__(256, 2) lin_gemm_wide(const bf16* __restrict__ x, int ldx, int M, int K, Seg2 s,
                                                        SeqRows sq) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int rt = SEQ ? blockIdx.x : blockIdx.y, nt = SEQ ? blockIdx.y : blockIdx.x;
  if constexpr (SEQ) {
    const int b = blockIdx.z;
    M = sq.len[b];
    if (rt * WM >= M) return;   // whole workgroup, before any barrier
    x += sq.off[b] * (int64_t)ldx;
    s.y1 = (bf16*)s.y1 + b * sq.y_bstride;
    s.y2 = (bf16*)s.y2 + b * sq.y_bstride;
  }
  const int m0 = rt * WM, n0 = nt * WN;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const uint32_t lds0 = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, smem);
  // loader: the stage holds WM rows of x then WN weight rows; wave w fills rows
  // (WM + WN) / 4 * w .. +95, 16 rows (1 KB) per load; lane l writes slot l % 4 of its row and so
  // loads logical piece wslot(l % 4, row)
  const bf16* gp[WLOADS];
#pragma unroll
  for (int k = 0; k < WLOADS; ++k) {
    const int r = (WM + WN) / 4 * w + 16 * k + (lane >> 2);
    const int piece = wslot(lane & 3, r);
    gp[k] = r < WM ? x + (size_t)min(m0 + r, M - 1) * ldx + 8 * piece
                   : wrow<bf16>(s, min(n0 + r - WM, s.n - 1), K) + 8 * piece;
  }
  auto issue = [&](int kt) {
    const uint32_t base = lds0 + (kt % WSTAGES) * WBUF + ((WM + WN) / 4 * w) * WROW;
#pragma unroll
    for (int k = 0; k < WLOADS; ++k) dma16(gp[k] + kt * WK, __builtin_amdgcn_readfirstlane(base + k * 1024));
  };
  f32x16e acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16e{};
  const int wm = 128 * (w >> 1), wn = 64 * (w & 1);
  const int NK = K / WK;
  issue(0);
  if (NK > 1) issue(1);
  for (int kt = 0; kt < NK; ++kt) {
    if (kt + 1 < NK)   // step kt landed; step kt + 1 may still be in flight
      wait_loads<WLOADS>();
    else
      wait_loads<0>();
    lds_barrier();   // everyone's loads of step kt are in; step kt - 1's stage is no longer read
    if (kt + 2 < NK) issue(kt + 2);   // into the stage of step kt - 1
    const unsigned char* A = smem + (kt % WSTAGES) * WBUF;
    const unsigned char* B = A + WM * WROW;
    // all 12 fragments of the step are read first, then the 16 MFMAs
    bf16x8e af[WK / 16][4], bfr[WK / 16][2];
#pragma unroll
    for (int ks = 0; ks < WK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm + 32 * i + l32;
        af[ks][i] = *reinterpret_cast<const bf16x8e*>(A + r * WROW + 16 * wslot(2 * ks + g, r));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn + 32 * j + l32;
        bfr[ks][j] = *reinterpret_cast<const bf16x8e*>(B + r * WROW + 16 * wslot(2 * ks + g, r));
      }
    }
#pragma unroll
    for (int ks = 0; ks < WK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks][j], af[ks][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);   // the 12 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // then the 16 MFMAs
  }
  // D^T block (i, j): lane holds output row m = wm + 32 i + l32, columns wn + 32 j + 8 q + 4 g + e
  __syncthreads();   // every wave is done with the operand stages (no load is in flight)
  bf16* Cs = reinterpret_cast<bf16*>(smem);   // [WM][WCS]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[i][j][4 * q + e];
        *reinterpret_cast<bf16x4*>(Cs + (wm + 32 * i + l32) * WCS + wn + 32 * j + 8 * q + 4 * g) = v;
      }
  __syncthreads();
  const int c = t & 15;
#pragma unroll 4
  for (int k = 0; k < WM / 16; ++k) {
    const int r = (t >> 4) + 16 * k;
    const int m = m0 + r, n = n0 + 8 * c;
    if (m < M && n < s.n) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(Cs + r * WCS + 8 * c);
      bf16* dst;
      if (SEQ && sq.head_stride > 0) {   // the tile's 128 columns are one head: one contiguous 64 KB block
        const int nn = n < s.n1 ? n : n - s.n1;
        dst = (n < s.n1 ? (bf16*)s.y1 : (bf16*)s.y2) + (size_t)(nn >> 7) * sq.head_stride + (size_t)m * 128 + (nn & 127);
      } else {
        dst = n < s.n1 ? (bf16*)s.y1 + (size_t)m * s.ldy1 + n : (bf16*)s.y2 + (size_t)m * s.ldy2 + (n - s.n1);
      }
      *reinterpret_cast<i32x4*>(dst) = v;
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// the staged GEMM epilogue writes 8 consecutive bf16 outputs per 16-byte store
bool staged_ok(const Seg2& s) {
  const bool two = s.n != s.n1;
  return s.n % 8 == 0 && s.n1 % 8 == 0 && s.ldy1 % 8 == 0 && aligned16(s.y1) &&
         (!two || (s.ldy2 % 8 == 0 && aligned16(s.y2)));
}

// The matrix-vector kernel for M < kGemmMinRows rows of bf16 x over up to three segments, and
// with `fin` the kv finish in one extra column of workgroups. Two weight rows per wave for wide
// outputs (each wave reads x once for both: W_O, 7168 x 16384, takes 45.3 us with W_UV against
// 47.4 us at one row per wave); K split over 2 or 4 waves until about 16 waves per CU have work, as
// long as every lane keeps at least 2 pieces of each row.
hipError_t gemv(const bf16* x, int ldx, int M, int K, const Seg3& s, const KvFinish* fin, hipStream_t stream) {
  const int n = s.end[2];
  const int rw = n >= 4096 ? 2 : 1;
  const int64_t row_waves = (n + rw - 1) / rw;
  int ks = 1;
  while (ks < 4 && row_waves * ks < 4096 && K / 8 >= 64 * 2 * (2 * ks)) ks *= 2;
  const int rb = M == 1 ? 1 : (M == 2 ? 2 : 4);
  const int rows_per_wg = rw * 4 / ks;
  const dim3 grid((n + rows_per_wg - 1) / rows_per_wg + (fin != nullptr ? 1 : 0), (M + rb - 1) / rb);
  const KvFinish none{nullptr, nullptr, nullptr, nullptr, nullptr, 0.0f, 0, 1, 0, 0, 0.0};
  const KvFinish& fk = fin != nullptr ? *fin : none;
#define MLA_LIN_GEMV_F(RW, KS, F)                                                                                \
  do {                                                                                                           \
    if (rb == 1)                                                                                                 \
      hipLaunchKernelGGL((lin_gemv<RW, 1, KS, F>), grid, dim3(256), 0, stream, x, ldx, M, K, s, fk);             \
    else if (rb == 2)                                                                                            \
      hipLaunchKernelGGL((lin_gemv<RW, 2, KS, F>), grid, dim3(256), 0, stream, x, ldx, M, K, s, fk);             \
    else                                                                                                         \
      hipLaunchKernelGGL((lin_gemv<RW, 4, KS, F>), grid, dim3(256), 0, stream, x, ldx, M, K, s, fk);             \
  } while (0)
#define MLA_LIN_GEMV(RW, KS)          \
  do {                                \
    if (fin != nullptr)               \
      MLA_LIN_GEMV_F(RW, KS, true);   \
    else                              \
      MLA_LIN_GEMV_F(RW, KS, false);  \
  } while (0)
  if (rw == 1) {
    if (ks == 1) MLA_LIN_GEMV(1, 1); else if (ks == 2) MLA_LIN_GEMV(1, 2); else MLA_LIN_GEMV(1, 4);
  } else {
    if (ks == 1) MLA_LIN_GEMV(2, 1); else if (ks == 2) MLA_LIN_GEMV(2, 2); else MLA_LIN_GEMV(2, 4);
  }
#undef MLA_LIN_GEMV
#undef MLA_LIN_GEMV_F
  return hipGetLastError();
}

// y = x W^T over the two segments; Ty is float or the storage type T
template <typename T, typename Ty>
hipError_t linear(const T* x, int ldx, int M, int K, const Seg2& s, hipStream_t stream) {
  if (M <= 0 || s.n <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    const bool vec = K % 8 == 0 && ldx % 8 == 0 && aligned16(x) && aligned16(s.w1) && (s.n == s.n1 || aligned16(s.w2));
    if constexpr (sizeof(Ty) == 2) {
      if (vec && M >= WM && K % WK == 0 && staged_ok(s)) {
        static std::atomic<uint32_t> wide_lds_set{0};
        const hipError_t e = ensure_lds_limit(wide_lds_set, {{(const void*)lin_gemm_wide<false>, WIDE_LDS}});
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((lin_gemm_wide<false>), dim3((s.n + WN - 1) / WN, (M + WM - 1) / WM), dim3(256), WIDE_LDS,
                           stream, x, ldx, M, K, s, SeqRows{nullptr, nullptr, 0});
        return hipGetLastError();
      }
    }
    if (vec && M >= kGemmMinRows && K % TK == 0) {
      static std::atomic<uint32_t> lds_set{0};
      const hipError_t e = ensure_lds_limit(lds_set, {{(const void*)lin_gemm<Ty, false, false>, GEMM_LDS},
                                                      {(const void*)lin_gemm<Ty, false, sizeof(Ty) == 2>, GEMM_LDS}});
      if (e != hipSuccess) return e;
      const dim3 grid((s.n + TN - 1) / TN, (M + TM - 1) / TM);
      if (sizeof(Ty) == 2 && staged_ok(s))
        hipLaunchKernelGGL((lin_gemm<Ty, false, sizeof(Ty) == 2>), grid, dim3(256), GEMM_LDS, stream, x, ldx, M, K, s,
                           SeqRows{nullptr, nullptr, 0});
      else
        hipLaunchKernelGGL((lin_gemm<Ty, false, false>), grid, dim3(256), GEMM_LDS, stream, x, ldx, M, K, s,
                           SeqRows{nullptr, nullptr, 0});
      return hipGetLastError();
    }
    if (vec && M < kGemmMinRows) {
      const int f = sizeof(Ty) == 4 ? 1 : 0;
      const Seg3 s3{{s.w1, s.w2, s.w2}, {s.y1, s.y2, s.y2}, {s.n1, s.n, s.n}, {s.ldy1, s.ldy2, s.ldy2}, {f, f, f}};
      return gemv(x, ldx, M, K, s3, nullptr, stream);
    }
  }
  hipLaunchKernelGGL((lin_generic<T, Ty>), dim3((s.n + 3) / 4, M < 65535 ? M : 65535), dim3(256), 0, stream, x, ldx,
                     M, K, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- kv finish
// One block per new token (grid (n_new, batch)): finish_token on the token's float32 projection.
template <typename T>
__global__ void __launch_bounds__(256) kv_finish(KvFinish f) {
  __shared__ float red[4];
  finish_token<T>(f, blockIdx.y * f.n_new + blockIdx.x, red);
}

}  // namespace lin

size_t project_workspace_bytes(const LayerDims& L, int n_rows, int d_q, int elem_bytes) {
  const size_t kv = (size_t)n_rows * (L.d_latent + L.d_rope) * sizeof(float);
  const size_t q = (size_t)n_rows * d_q * elem_bytes;
  size_t b = kv > q ? kv : q;
  return (b + 255) & ~(size_t)255;
}

template <typename T>
hipError_t launch_project_kv_append(const LayerDims& L, int batch, int n_new, int d_model, const void* h,
                                    const void* w_dkv, const void* w_kr, const void* norm_w, float eps, int use_norm,
                                    void* cache, const int64_t* seq_off, const int32_t* len_before, void* workspace,
                                    hipStream_t stream) {
  const int row = L.d_latent + L.d_rope;
  float* pre = (float*)workspace;
  lin::Seg2 s{w_dkv, w_kr, pre, pre + L.d_latent, L.d_latent, row, row, row};
  hipError_t e = lin::linear<T, float>((const T*)h, d_model, batch * n_new, d_model, s, stream);
  if (e != hipSuccess) return e;
  const lin::KvFinish f{pre, norm_w, cache, seq_off, len_before, eps, use_norm, n_new, L.d_latent, L.d_rope,
                        L.rope_base};
  hipLaunchKernelGGL(lin::kv_finish<T>, dim3(n_new, batch), dim3(256), 0, stream, f);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_project_q(const LayerDims& L, int n_rows, int d_model, int d_q, const void* h, const void* w_dq,
                            const void* w_uq, const void* w_qr, void* q_nope, void* q_rope, void* workspace,
                            hipStream_t stream) {
  const T* x = (const T*)h;
  int K = d_model;
  if (d_q > 0) {
    lin::Seg2 s{w_dq, nullptr, workspace, nullptr, d_q, d_q, d_q, 0};
    hipError_t e = lin::linear<T, T>(x, d_model, n_rows, d_model, s, stream);
    if (e != hipSuccess) return e;
    x = (const T*)workspace;
    K = d_q;
  }
  const int n1 = L.n_heads * L.d_nope, n2 = L.n_heads * L.d_rope;
  lin::Seg2 s{w_uq, w_qr, q_nope, q_rope, n1, n1 + n2, n1, n2};
  return lin::linear<T, T>(x, K, n_rows, K, s, stream);
}

size_t project_inputs_workspace_bytes(const LayerDims& L, int n_rows, int d_q, int elem_bytes) {
  const size_t kv = ((size_t)n_rows * (L.d_latent + L.d_rope) * sizeof(float) + 255) & ~(size_t)255;
  return kv + (((size_t)n_rows * d_q * elem_bytes + 255) & ~(size_t)255);
}

// Both projections of the layer input: with few rows of bf16 in the layouts the matrix-vector
// kernel takes, two launches instead of four. The first reads h once for W_DKV, W_KR and W_DQ
// (three segments: the kv projection in float32, c_Q rounded to bf16); the second runs W_UQ and
// W_QR over c_Q (or over h without query compression) with the kv finish in one extra column of
// workgroups. Otherwise the two calls' own launches, on the two halves of the workspace.
template <typename T>
hipError_t launch_project_inputs(const LayerDims& L, int batch, int n_new, int d_model, int d_q, const void* h,
                                 const void* w_dkv, const void* w_kr, const void* norm_w, float eps, int use_norm,
                                 void* cache, const int64_t* seq_off, const int32_t* len_before, const void* w_dq,
                                 const void* w_uq, const void* w_qr, void* q_nope, void* q_rope, void* workspace,
                                 hipStream_t stream) {
  const int rows = batch * n_new;
  const int row = L.d_latent + L.d_rope;
  float* pre = (float*)workspace;
  void* cq = (char*)workspace + (((size_t)rows * row * sizeof(float) + 255) & ~(size_t)255);
  const auto al = [](const void* p) { return p == nullptr || lin::aligned16(p); };
  const bool fused = sizeof(T) == 2 && rows < kGemmMinRows && lin::aligned16(h) && d_model % 8 == 0 && d_q % 8 == 0 &&
                     al(w_dkv) && al(w_kr) && al(w_dq) && al(w_uq) && al(w_qr);
  if (!fused) {
    hipError_t e = launch_project_kv_append<T>(L, batch, n_new, d_model, h, w_dkv, w_kr, norm_w, eps, use_norm, cache,
                                               seq_off, len_before, pre, stream);
    if (e != hipSuccess) return e;
    return launch_project_q<T>(L, rows, d_model, d_q, h, w_dq, w_uq, w_qr, q_nope, q_rope, cq, stream);
  }
  const lin::Seg3 s1{{w_dkv, w_kr, w_dq}, {pre, pre + L.d_latent, cq}, {L.d_latent, row, row + d_q}, {row, row, d_q},
                     {1, 1, 0}};
  hipError_t e = lin::gemv((const bf16*)h, d_model, rows, d_model, s1, nullptr, stream);
  if (e != hipSuccess) return e;
  const int n1 = L.n_heads * L.d_nope, n2 = L.n_heads * L.d_rope;
  const lin::Seg3 s2{{w_uq, w_qr, w_qr}, {q_nope, q_rope, q_rope}, {n1, n1 + n2, n1 + n2}, {n1, n2, n2}, {0, 0, 0}};
  const lin::KvFinish f{pre, norm_w, cache, seq_off, len_before, eps, use_norm, n_new, L.d_latent, L.d_rope,
                        L.rope_base};
  const bf16* x2 = d_q > 0 ? (const bf16*)cq : (const bf16*)h;
  const int k2 = d_q > 0 ? d_q : d_model;
  return lin::gemv(x2, k2, rows, k2, s2, &f, stream);
}

template <typename T>
hipError_t launch_linear(const void* x, int ldx, int M, int K, const void* w, int N, void* y, int ldy,
                         hipStream_t stream) {
  lin::Seg2 s{w, nullptr, y, nullptr, N, N, ldy, 0};
  return lin::linear<T, T>((const T*)x, ldx, M, K, s, stream);
}
template hipError_t launch_linear<float>(const void*, int, int, int, const void*, int, void*, int, hipStream_t);
template hipError_t launch_linear<__bf16>(const void*, int, int, int, const void*, int, void*, int, hipStream_t);

// K_C = C W_UK^T and V = C W_UV^T for every key of every sequence (the explicit form's key and
// value reconstruction): per sequence b the latents are the first d_latent columns of its cache
// rows seq_off[b] .. seq_off[b] + seq_len[b] - 1; outputs kc / vv head-major,
// [batch][H][max_seq_len][128], so that the attention's key/value tiles of one head are contiguous.
hipError_t launch_kv_expand(int batch, int max_seq_len, int n_out, int d_latent, int row, const void* cache,
                            const int64_t* seq_off, const int32_t* seq_len, const void* w_uk, const void* w_uv,
                            void* kc, void* vv, hipStream_t stream) {
  static std::atomic<uint32_t> lds_set{0};
  {
    const hipError_t e = ensure_lds_limit(lds_set, {{(const void*)lin::lin_gemm_wide<true>, lin::WIDE_LDS}});
    if (e != hipSuccess) return e;
  }
  lin::Seg2 s{w_uk, w_uv, kc, vv, n_out, 2 * n_out, n_out, n_out};
  lin::SeqRows sq{seq_len, seq_off, (int64_t)max_seq_len * n_out, (int64_t)max_seq_len * 128};
  // n_out = H * 128 and the workspace rows keep every staged 16-byte store aligned; d_latent = 512
  // is a whole number of K steps
  const dim3 grid((max_seq_len + lin::WM - 1) / lin::WM, (2 * n_out + lin::WN - 1) / lin::WN, batch);
  hipLaunchKernelGGL((lin::lin_gemm_wide<true>), grid, dim3(256), lin::WIDE_LDS, stream, (const bf16*)cache,
                     row, max_seq_len, d_latent, s, sq);
  return hipGetLastError();
}

template hipError_t launch_project_kv_append<float>(const LayerDims&, int, int, int, const void*, const void*,
                                                    const void*, const void*, float, int, void*, const int64_t*,
                                                    const int32_t*, void*, hipStream_t);
template hipError_t launch_project_kv_append<__bf16>(const LayerDims&, int, int, int, const void*, const void*,
                                                     const void*, const void*, float, int, void*, const int64_t*,
                                                     const int32_t*, void*, hipStream_t);
template hipError_t launch_project_inputs<float>(const LayerDims&, int, int, int, int, const void*, const void*,
                                                 const void*, const void*, float, int, void*, const int64_t*,
                                                 const int32_t*, const void*, const void*, const void*, void*, void*,
                                                 void*, hipStream_t);
template hipError_t launch_project_inputs<__bf16>(const LayerDims&, int, int, int, int, const void*, const void*,
                                                  const void*, const void*, float, int, void*, const int64_t*,
                                                  const int32_t*, const void*, const void*, const void*, void*, void*,
                                                  void*, hipStream_t);
template hipError_t launch_project_q<float>(const LayerDims&, int, int, int, const void*, const void*, const void*,
                                            const void*, void*, void*, void*, hipStream_t);
template hipError_t launch_project_q<__bf16>(const LayerDims&, int, int, int, const void*, const void*, const void*,
                                             const void*, void*, void*, void*, hipStream_t);

}  // namespace mla
