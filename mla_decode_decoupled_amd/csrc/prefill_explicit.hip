// Non-absorbed (explicit-key) attention for chunked prefill, DeepSeek-V2/V3 head shape
// (d_nope = d_v = 128, d_rope = 64, d_latent = 512, bf16), any head count.
//
// The absorbed form scores 576-wide latent rows and sums 512-wide latents for every (query row,
// key) pair, 2 H (576 + 512) flops per pair. With many query rows per sequence it is cheaper to
// go back to the explicit form the pages start from ("Decoupled RoPE · MLA Part 2", §2.1: rebuild
// the content key K_C = W_UK c and the value V = W_UV c, and §3.2: concatenate the shared rotated
// position key to every head's content key; "从零理解 MLA", the non-absorbed forward before
// section "矩阵吸收"): rebuild K_C and V once per key (a GEMM over the cached latents), then run
// ordinary multi-head attention with 192-wide keys and 128-wide values, 2 H (192 + 128) flops per
// pair, and produce the heads' outputs o directly.
//
// attn_explicit: one workgroup per (sequence b, head i, block of 128 query rows); 4 waves of 32
// query rows each walk the visible keys in tiles of 32, the tiles staged in LDS for all 4 waves
// (global -> registers -> LDS, double-buffered: the next tile's loads are in flight during the
// current tile's MFMAs). Per wave and tile:
//   * scores S^T [32 keys x 32 rows] = K Q^T with 12 MFMA 32x32x16 over the 192 dims; the query
//     fragments (content part, and the position part rotated on load) stay in registers. The key
//     rows of the A operand are taken in a permuted order so that each lane's 16 score registers
//     are exactly the keys its P.V B operand needs (P never leaves the registers);
//   * online softmax per query row in log2 units (running max, rescaled sum and accumulator),
//     keys past the row's causal limit masked;
//   * O^T [128 x 32 rows] += V^T P^T with 8 MFMAs, V^T read from the row-major value tile with the
//     gfx950 transpose read ds_read_b64_tr_b16.
// The (sequence, head) pairs are dealt so that all query blocks of one pair run on the same XCD
// and share its L2 for the key/value tiles, and the blocks with the most keys start first.
#include <cstddef>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace xp {

constexpr int DN = 128;               // content key / query width
constexpr int DR = 64;                // position width
constexpr int DK = DN + DR;           // 192
constexpr int DV = 128;
constexpr int DC = 512;
constexpr int ROW = DC + DR;          // cache row, 576
constexpr int BM = 128;               // query rows per workgroup (4 waves x 32)
constexpr int TK = 32;                // keys per tile
constexpr float RESCALE = 8.0f;       // log2 units a score may exceed the running reference
// LDS has 64 banks of 4 bytes. Key rows of 400 bytes (= 144 mod 256) put the 16-byte reads of 16
// consecutive rows on 16 different bank groups; value rows of 320 bytes (= 64 mod 256) give the
// transpose reads (4 rows x 64 bytes per 32 lanes) 256 distinct bytes.
constexpr int KS_STRIDE = DK + 8;     // bf16 per staged key row (400 bytes)
constexpr int VS_STRIDE = DV + 32;    // bf16 per staged value row (320 bytes)
constexpr int KS_ELEMS = TK * KS_STRIDE;
constexpr int VS_ELEMS = TK * VS_STRIDE;
constexpr int BUF_ELEMS = KS_ELEMS + VS_ELEMS;
constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;   // two buffers
// 16-byte pieces per tile: content keys 32 x 16, position keys 32 x 8, values 32 x 16
constexpr int PIECES = TK * (DN / 8) + TK * (DR / 8) + TK * (DV / 8);   // 1280
constexpr int PIECES_PER_THREAD = PIECES / 256;                          // 5
static_assert(PIECES % 256 == 0, "tile must split evenly over the workgroup");

typedef __bf16 bf16x8e __attribute__((ext_vector_type(8)));
typedef short i16x4e __attribute__((ext_vector_type(4)));
typedef float f32x16e __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
typedef float f32x2e __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16e mfma(bf16x8e a, bf16x8e b, f32x16e c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A-operand row r of the score MFMA holds key pi(r) of the tile, pi(8j + 4g + i) =
// 16 (j / 2) + 8 g + 4 (j % 2) + i, so that the lane of key half g finds keys 8g .. 8g+7 in its
// score registers 0..7 and keys 16+8g .. 16+8g+7 in registers 8..15: its two P.V B fragments.
__device__ __forceinline__ int key_of_row(int r) {
  const int j = r >> 3, g = (r >> 2) & 1, i = r & 3;
  return 16 * (j >> 1) + 8 * g + 4 * (j & 1) + i;
}

// grid: batch * H * ceil(n_q / BM) workgroups, 256 threads, LDS_BYTES dynamic LDS.
__global__ void __launch_bounds__(256, 2) attn_explicit(const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
                                                     const bf16* __restrict__ cache, const int64_t* __restrict__ seq_off,
                                                     const int32_t* __restrict__ seq_len, const bf16* __restrict__ kc,
                                                     const bf16* __restrict__ vv, int H, int n_q, int max_seq_len,
                                                     int n_qb, double base, float scale_log2, bf16* __restrict__ o,
                                                     float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* smem = reinterpret_cast<bf16*>(smem_raw);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // workgroup -> (pair = b * H + i, query block), all blocks of a pair on one XCD, heaviest first
  const int pairs = gridDim.x / n_qb;
  int pair, qb;
  {
    const int wg = blockIdx.x;
    if (pairs % 8 == 0) {
      const int x = wg & 7, k = wg >> 3;
      pair = (k / n_qb) * 8 + x;
      qb = n_qb - 1 - (k % n_qb);
    } else {
      pair = wg / n_qb;
      qb = n_qb - 1 - (wg % n_qb);
    }
  }
  const int b = pair / H, i = pair % H;
  const int S = seq_len[b];
  const int64_t off = seq_off[b];
  const int t0 = qb * BM;                    // first query row of the workgroup
  const int row = t0 + 32 * w + l32;         // this lane's query row (the B / accumulator column)
  const bool row_ok = row < n_q;
  const int pos = S - n_q + (row_ok ? row : n_q - 1);   // its position = last visible key
  const int wave_pos0 = S - n_q + t0 + 32 * w;           // position of the wave's first row
  // keys the workgroup needs: up to the last row's position
  const int last_row = min(t0 + BM, n_q) - 1;
  const int n_keys = S - n_q + last_row + 1;
  const int n_tiles = (n_keys + TK - 1) / TK;

  // ---- query fragments: dims 16 s + 8 g .. +7 of this lane's row; s < 8 content, s >= 8 position
  bf16x8e qf[12];
  {
    const size_t qr = ((size_t)b * n_q + (row_ok ? row : 0)) * H + i;
    const bf16* qn = q_nope + qr * DN;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8e*>(qn + 16 * s + 8 * g);
    const bf16* qp = q_rope + qr * DR;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8e raw = *reinterpret_cast<const bf16x8e*>(qp + 16 * s + 8 * g);
      bf16x8e rot;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 8 * s + 4 * g + e;   // pair (2j, 2j+1)
        float sn, cs;
        rope_sincos(rope_theta(base, j, DR), pos, &sn, &cs);
        const float x0 = (float)raw[2 * e], x1 = (float)raw[2 * e + 1];
        rot[2 * e] = (bf16)(x0 * cs - x1 * sn);
        rot[2 * e + 1] = (bf16)(x0 * sn + x1 * cs);
      }
      qf[8 + s] = rot;
    }
  }

  // ---- tile loader: per thread t, two 16-byte pieces of content keys (key t / 16 and 16 + t / 16,
  // chunk t % 16), one of position keys (key t / 8, chunk t % 8) and two of values (as the content
  // keys); keys past the sequence re-read its last key (they are masked)
  static_assert(PIECES_PER_THREAD == 5, "loader layout");
  const size_t kvrow0 = (size_t)b * max_seq_len;
  const int tk = threadIdx.x >> 4, tc = threadIdx.x & 15;     // content keys / values
  const int rk = threadIdx.x >> 3, rc = threadIdx.x & 7;      // position keys
  i32x4 ldA[PIECES_PER_THREAD], ldB[PIECES_PER_THREAD];   // two register sets: tiles t+1 and t+2 in flight
  // whole tiles advance three base pointers; only the sequence's last, partial tile clamps keys
  const bf16* kc_p = kc + ((kvrow0 + tk) * H + i) * DN + 8 * tc;
  const bf16* vv_p = vv + ((kvrow0 + tk) * H + i) * DV + 8 * tc;
  const bf16* kr_p = cache + (off + rk) * ROW + DC + 8 * rc;
  const size_t kv_step = (size_t)TK * H * DN;   // one tile of keys in kc / vv
  auto gload = [&](i32x4 (&ld)[PIECES_PER_THREAD], int tile) {
    const int j0 = tile * TK;
    if (j0 + TK <= S) {
      const size_t o = (size_t)tile * kv_step;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ld[h] = *reinterpret_cast<const i32x4*>(kc_p + o + (size_t)16 * h * H * DN);
        ld[3 + h] = *reinterpret_cast<const i32x4*>(vv_p + o + (size_t)16 * h * H * DV);
      }
      ld[2] = *reinterpret_cast<const i32x4*>(kr_p + (size_t)j0 * ROW);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = min(j0 + tk + 16 * h, S - 1);
        ld[h] = *reinterpret_cast<const i32x4*>(kc + ((kvrow0 + key) * H + i) * DN + 8 * tc);
        ld[3 + h] = *reinterpret_cast<const i32x4*>(vv + ((kvrow0 + key) * H + i) * DV + 8 * tc);
      }
      ld[2] = *reinterpret_cast<const i32x4*>(cache + (off + min(j0 + rk, S - 1)) * ROW + DC + 8 * rc);
    }
  };
  auto lstore = [&](const i32x4 (&ld)[PIECES_PER_THREAD], int buf) {
    bf16* ks = smem + buf * BUF_ELEMS;
    bf16* vs = ks + KS_ELEMS;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<i32x4*>(ks + (tk + 16 * h) * KS_STRIDE + 8 * tc) = ld[h];
      *reinterpret_cast<i32x4*>(vs + (tk + 16 * h) * VS_STRIDE + 8 * tc) = ld[3 + h];
    }
    *reinterpret_cast<i32x4*>(ks + rk * KS_STRIDE + DN + 8 * rc) = ld[2];
  };

  f32x16e oacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) oacc[c] = f32x16e{};
  float m_run = -INFINITY, l_run = 0.0f;
  const int akey = key_of_row(l32);

  // Tile t is in LDS buffer t % 2 while the registers hold tiles t + 1 and t + 2 in flight (two
  // sets, alternating), so a tile's global loads have two iterations to land before they are
  // stored to LDS at the end of the iteration before its own.
  auto compute = [&](int t) {
    const int buf = t & 1;
    const bf16* ks = smem + buf * BUF_ELEMS;
    const bf16* vs = ks + KS_ELEMS;
    // scores of the tile: A = key rows (permuted), B = this wave's query fragments
    // all 12 key fragments are read before the first MFMA, so the chain waits for one LDS round trip
    f32x16e sacc = f32x16e{};
    const bf16* krow = ks + akey * KS_STRIDE + 8 * g;
    bf16x8e kf[12];
#pragma unroll
    for (int s = 0; s < 6; ++s) kf[s] = *reinterpret_cast<const bf16x8e*>(krow + 16 * s);
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      sacc = mfma(kf[s], qf[s], sacc);
      if (s + 6 < 12) kf[s + 6] = *reinterpret_cast<const bf16x8e*>(krow + 16 * (s + 6));
    }
    // six reads ahead of the chain, then one read behind each MFMA (it reuses the registers the
    // MFMA has just consumed), then the last six MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    // causal mask and online softmax on the raw scores (the scale is positive, so it is applied in
    // the exponent); register r holds key 16 (r / 8) + 8 g + (r % 8). Only tiles reaching past the
    // first position of the wave's rows need the mask.
    const int j0 = t * TK;
    float sv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
    if (j0 + TK - 1 > wave_pos0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j0 + 16 * (r >> 3) + 8 * g + (r & 7) > pos) sv[r] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    // Lazy rescaling: the running reference m_run only moves when a score exceeds it by more than
    // RESCALE (log2 units), so probabilities stay below 2^RESCALE and the accumulator is rescaled
    // only on those (rare, mostly early) tiles. Softmax is exact for any reference. Key 0 is
    // visible to every row, so the first tile always sets a finite reference.
    if (__any(mx > m_run + RESCALE)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c) oacc[c] *= alpha;
      m_run = m_new;
    }
    int pk[8];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[r], scale_log2, -m_run));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[r + 1], scale_log2, -m_run));
      psum += p0 + p1;
      pk[r / 2] = __builtin_bit_cast(int, __builtin_convertvector((f32x2e){p0, p1}, bf16x2e));
    }
    l_run += psum;
    const int pk0[4] = {pk[0], pk[1], pk[2], pk[3]}, pk1[4] = {pk[4], pk[5], pk[6], pk[7]};
    const bf16x8e pb[2] = {__builtin_bit_cast(bf16x8e, pk0), __builtin_bit_cast(bf16x8e, pk1)};
    // O^T += V^T P^T: A fragment of col block c, key step s = value rows 16 s + 8 g .. +7 of column
    // 32 c + l32, gathered by two transpose reads (lane L of a 16-lane group points at row
    // 16 s + 8 g + 4 h + L / 4, columns 32 c + 16 (q & 1) + 4 (L & 3) .. +3, q = lane / 16)
    const int q = lane >> 4, L = lane & 15;
    bf16x8e vf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        i16x4e hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16* p = vs + (16 * s + 8 * g + 4 * h + (L >> 2)) * VS_STRIDE + 32 * c + 16 * (q & 1) + 4 * (L & 3);
          hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4e*)MLA_LDS(bf16, p));
        }
        vf[s][c] = __builtin_bit_cast(bf16x8e, hv);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) oacc[c] = mfma(vf[s][c], pb[s], oacc[c]);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };
  gload(ldA, 0);
  if (n_tiles > 1) gload(ldB, 1);
  lstore(ldA, 0);
  __syncthreads();
  for (int t = 0; t < n_tiles; t += 2) {
    // even tile: set A is free (tile t was stored), set B holds tile t + 1
    if (t + 2 < n_tiles) gload(ldA, t + 2);
    compute(t);
    if (t + 1 >= n_tiles) break;
    lstore(ldB, (t + 1) & 1);   // buffer (t + 1) % 2 was last read in iteration t - 1
    __syncthreads();
    // odd tile: set B is free, set A holds tile t + 2
    if (t + 3 < n_tiles) gload(ldB, t + 3);
    compute(t + 1);
    if (t + 2 >= n_tiles) break;
    lstore(ldA, t & 1);
    __syncthreads();
  }
  // ---- output: o[row][32 c + 8 r4 + 4 g + e] = O^T / l, four consecutive values per store
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = 1.0f / l_tot;
  bf16* orow = o + (((size_t)b * n_q + row) * H + i) * DV;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16)(oacc[c][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * c + 8 * r4 + 4 * g) = v4;
    }
  if (lse != nullptr && g == 0) lse[((size_t)b * n_q + row) * H + i] = (m_run + log2f(l_tot)) * kLn2;
}

}  // namespace xp

bool prefill_explicit_supported(const LayerDims& L) {
  return L.d_nope == xp::DN && L.d_rope == xp::DR && L.d_v == xp::DV && L.d_latent == xp::DC;
}

size_t prefill_explicit_workspace_bytes(const LayerDims& L, int batch, int max_seq_len) {
  return (size_t)2 * batch * max_seq_len * L.n_heads * xp::DN * sizeof(bf16);
}

hipError_t launch_prefill_explicit(const LayerDims& L, int batch, int n_q, const void* q_nope, const void* q_rope,
                                   const void* cache, const int64_t* seq_off, const int32_t* seq_len, int max_seq_len,
                                   const void* w_uk, const void* w_uv, void* workspace, void* o, float* lse,
                                   hipStream_t stream) {
  const int H = L.n_heads;
  bf16* kc = (bf16*)workspace;
  bf16* vv = kc + (size_t)batch * max_seq_len * H * xp::DN;
  hipError_t e = launch_kv_expand(batch, max_seq_len, H * xp::DN, xp::DC, xp::ROW, cache, seq_off, seq_len, w_uk,
                                  w_uv, kc, vv, stream);
  if (e != hipSuccess) return e;
  static bool attr_set = false;
  if (!attr_set) {
    e = hipFuncSetAttribute((const void*)xp::attn_explicit, hipFuncAttributeMaxDynamicSharedMemorySize, xp::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_qb = (n_q + xp::BM - 1) / xp::BM;
  hipLaunchKernelGGL(xp::attn_explicit, dim3(batch * H * n_qb), dim3(256), xp::LDS_BYTES, stream, (const bf16*)q_nope,
                     (const bf16*)q_rope, (const bf16*)cache, seq_off, seq_len, (const bf16*)kc, (const bf16*)vv, H, n_q,
                     max_seq_len, n_qb, L.rope_base, L.softmax_scale * kLog2e, (bf16*)o, lse);
  return hipGetLastError();
}

}  // namespace mla
