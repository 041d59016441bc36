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
// query rows each walk the visible keys in tiles of 32, the tiles staged in LDS for all 4 waves by
// direct 16-byte global -> LDS loads (five per wave and tile) into a ring of four buffers: two tiles
// in flight while the waves work on two. Per wave and tile:
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
// a lane's probability sum up to which no score can have moved the reference: 2^RESCALE / 2, half the
// bound, so that the rounding of the hardware exponential never hides a score just past the limit
constexpr float kRescaleSum = 128.0f;
// A staged tile: 32 key rows of 384 bytes (content key, then position key: 24 chunks of 16 bytes),
// then 32 value rows of 256 bytes (16 chunks), unpadded, as the direct loads write 1 KB runs. LDS
// has 64 banks of 4 bytes; the 16-byte chunks are permuted within each row (an XOR, its own
// inverse) so that both read patterns are conflict free:
//   key row r: chunk c sits at (c & ~7) | ((c ^ ((r >> 1) & 7)) & 7). The score reads take one chunk
//     of 16 keys that run over rows 0-15 or 16-31 (each half once); the 16 rows' (r & 1, (r >> 1) & 7)
//     are distinct, so their chunks land on 16 distinct groups of 4 banks (a row is 24 chunks,
//     8 mod 16);
//   value row r: chunk c sits at c ^ (4 (r & 3)). A transpose read takes 4 consecutive rows x 4
//     consecutive chunks per 32 lanes, which then cover all 16 bank groups.
constexpr int KROW = (DK * 2) / 16;   // 24 chunks per key row
constexpr int VROW = (DV * 2) / 16;   // 16 chunks per value row
constexpr int K_BYTES = TK * DK * 2;  // 12 KB
constexpr int BUF_BYTES = K_BYTES + TK * DV * 2;   // 20 KB
constexpr int NBUF = 4;
constexpr int LDS_BYTES = NBUF * BUF_BYTES;        // 80 KB: two workgroups per CU fill the 160 KB
constexpr int SLOTS = BUF_BYTES / 16;              // 1280 chunks per tile
constexpr int DMA_PER_WAVE = SLOTS / (4 * 64);     // 5 loads of 64 chunks per wave and tile
static_assert(SLOTS % 256 == 0 && (K_BYTES / 16) % 64 == 0, "every load is all key or all value chunks");
__device__ __forceinline__ int kchunk(int c, int r) { return (c & ~7) | ((c ^ (r >> 1)) & 7); }
__device__ __forceinline__ int vchunk(int c, int r) { return c ^ (4 * (r & 3)); }
// one 16-byte-per-lane direct global -> LDS load: lane l writes LDS bytes lds_base + 16 l
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vmcnt_5() { __builtin_amdgcn_s_waitcnt(5 | (7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_vmcnt_0() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }
// the max of v over lanes l and l ^ 32: v_permlane32_swap exchanges lanes 32-63 of its first
// operand with lanes 0-31 of its second, so with v in both the pair holds v[l] and v[l ^ 32]
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

  // ---- tile loader: load `it` of wave w moves chunks w * 320 + 64 it .. +63 of the tile (lane l one
  // of them): key chunks first (32 rows x 24), then value chunks (32 rows x 16). A lane reads the
  // logical chunk that the permutation puts at its LDS position, from a pointer that advances one
  // tile per load; in the sequence's last, partial tile, keys past its end re-read its last key
  // (they are masked).
  const size_t hrow0 = ((size_t)b * H + i) * max_seq_len;   // key 0 of this (sequence, head) in kc / vv
  const unsigned char* src[DMA_PER_WAVE];   // this lane's chunk in the next tile to load
  uint32_t stride[DMA_PER_WAVE];            // bytes from one key to the next (at most 32 KB)
  int srow[DMA_PER_WAVE];                   // the tile row (key) the lane loads
#pragma unroll
  for (int it = 0; it < DMA_PER_WAVE; ++it) {
    const int slot = w * (SLOTS / 4) + 64 * it + lane;
    if (slot < K_BYTES / 16) {
      const int r = slot / KROW, c = kchunk(slot % KROW, r);
      srow[it] = r;
      if (c < DN / 8) {   // content key chunk
        src[it] = reinterpret_cast<const unsigned char*>(kc + (hrow0 + r) * DN + 8 * c);
        stride[it] = DN * 2;
      } else {            // position key chunk, straight from the cache row (stored rotated)
        src[it] = reinterpret_cast<const unsigned char*>(cache + (off + r) * ROW + DC + 8 * (c - DN / 8));
        stride[it] = ROW * 2;
      }
    } else {
      const int v = slot - K_BYTES / 16, r = v / VROW, c = vchunk(v % VROW, r);
      srow[it] = r;
      src[it] = reinterpret_cast<const unsigned char*>(vv + (hrow0 + r) * DV + 8 * c);
      stride[it] = DV * 2;
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)MLA_LDS(unsigned char, smem_raw) +
                                                       w * (SLOTS / 4) * 16);
  // loads tile `tile` (the next one: tiles are loaded in order) into buffer `buf`
  size_t step_bytes[DMA_PER_WAVE];   // one tile of keys
#pragma unroll
  for (int it = 0; it < DMA_PER_WAVE; ++it) step_bytes[it] = (size_t)TK * stride[it];
  auto issue = [&](int tile, int buf) {
    const int j0 = tile * TK;
    if (j0 + TK <= S) {
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) dma16(src[it], lds0 + buf * BUF_BYTES + 1024 * it);
    } else {   // the last, partial tile (wave-uniform branch)
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) {
        const int over = max(0, j0 + srow[it] - (S - 1));
        dma16(src[it] - (size_t)over * stride[it], lds0 + buf * BUF_BYTES + 1024 * it);
      }
    }
#pragma unroll
    for (int it = 0; it < DMA_PER_WAVE; ++it) src[it] += step_bytes[it];
  };

  f32x16e oacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) oacc[c] = f32x16e{};
  float m_run = -INFINITY, l_run = 0.0f;
  const int akey = key_of_row(l32);
  // LDS read addresses, the same in every buffer (a buffer's offset is a constant of the unrolled
  // loop below):
  //   key k-step s reads logical chunk 2 s + g of row akey, at kchunk(2 s + g, akey): for s = 4 u + j
  //   that is kb[j] + 128 u (the permutation keeps each group of 8 chunks in place);
  //   value col block c of the transpose reads: row 16 s + 8 g + 4 h + L / 4 (its row & 3 = L / 4),
  //   logical chunk 4 c + 2 (q & 1) + (L & 3) / 2, byte 8 (L & 1): vb[c] + 256 (16 s + 4 h).
  const int q = lane >> 4, L = lane & 15;
  const unsigned char* kb[4];
  const unsigned char* vb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kb[j] = smem_raw + akey * (KROW * 16) + 16 * kchunk(2 * j + g, akey);
    vb[j] = smem_raw + K_BYTES + (8 * g + (L >> 2)) * (VROW * 16) +
            16 * vchunk(4 * j + 2 * (q & 1) + ((L & 3) >> 1), L >> 2) + 8 * (L & 1);
  }

  // scores of the tile in buffer `buf`: A = key rows (permuted), B = this wave's query fragments;
  // register r of the result holds key 16 (r / 8) + 8 g + (r % 8) of the tile
  auto scores = [&](int buf) {
    const int bo = buf * BUF_BYTES;
    f32x16e sacc = f32x16e{};
    bf16x8e kf[12];
#pragma unroll
    for (int s = 0; s < 6; ++s) kf[s] = *reinterpret_cast<const bf16x8e*>(kb[s & 3] + bo + 128 * (s >> 2));
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      sacc = mfma(kf[s], qf[s], sacc);
      if (s + 6 < 12) kf[s + 6] = *reinterpret_cast<const bf16x8e*>(kb[(s + 6) & 3] + bo + 128 * ((s + 6) >> 2));
    }
    return sacc;
  };
  // causal mask of tile t (only tiles reaching past the first position of the wave's rows need it)
  auto mask = [&](f32x16e& sv, int t) {
    const int j0 = t * TK;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (j0 + 16 * (r >> 3) + 8 * g + (r & 7) > pos) sv[r] = -INFINITY;
  };
  auto lane_max = [&](const f32x16e& sv) {
    float mx = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    return mx;
  };
  // P of the tile against the running reference (the scale is positive, so it is applied in the
  // exponent), packed as the two P.V B fragments; returns the sum of the lane's 16 probabilities
  auto probs = [&](const f32x16e& sv, bf16x8e* pb) {
    int pk[8];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[r], scale_log2, -m_run));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[r + 1], scale_log2, -m_run));
      psum += p0 + p1;
      pk[r / 2] = __builtin_bit_cast(int, __builtin_convertvector((f32x2e){p0, p1}, bf16x2e));
    }
    const int pk0[4] = {pk[0], pk[1], pk[2], pk[3]}, pk1[4] = {pk[4], pk[5], pk[6], pk[7]};
    pb[0] = __builtin_bit_cast(bf16x8e, pk0);
    pb[1] = __builtin_bit_cast(bf16x8e, pk1);
    return psum;
  };
  // O^T += V^T P^T for the tile in buffer `buf`: A fragment of col block c, key step s = value rows
  // 16 s + 8 g .. +7 of column 32 c + l32, gathered by two transpose reads
  auto pv = [&](int buf, const bf16x8e* pb) {
    const int bo = buf * BUF_BYTES;
    bf16x8e vf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        i16x4e hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned char* p = vb[c] + bo + (VROW * 16) * (16 * s + 4 * h);
          hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4e*)MLA_LDS(unsigned char, p));
        }
        vf[s][c] = __builtin_bit_cast(bf16x8e, hv);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) oacc[c] = mfma(vf[s][c], pb[s], oacc[c]);
  };
  // Lazy rescaling: the running reference m_run only moves when a score exceeds it by more than
  // RESCALE (log2 units), so probabilities stay below 2^RESCALE and the accumulator is rescaled
  // only on those (rare, mostly early) tiles. Softmax is exact for any reference. Key 0 is visible
  // to every row, so the first tile always sets a finite reference.
  // A tile's maximum is only needed when it may move the reference: if the sum of a lane's 16
  // probabilities against the current reference is at most kRescaleSum (< 2^RESCALE), none of them
  // reaches 2^RESCALE, so no score exceeds the reference by more than RESCALE and the rule would not
  // move it. Only a larger sum (rare) computes the maximum, applies the rule, and recomputes the
  // probabilities against the moved reference: the references, and so the results, are those of
  // taking every tile's maximum.
  auto rescale_to = [&](float mx) {
    if (__any(mx > m_run + RESCALE)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c) oacc[c] *= alpha;
      m_run = m_new;
    }
  };

  // Software pipeline, per iteration t: the score MFMAs of tile t + 1 run with the exponentials of
  // tile t between them; then the P.V MFMAs of tile t run with tile t + 1's row maxima between
  // them; then the reference moves if tile t + 1 needs it. Tile t sits in buffer t % 4, tiles t + 2
  // and t + 3 load into the other two. The last iteration scores a resident buffer once more and
  // discards it (its maximum is taken as -inf). The loop is unrolled by the 4 buffers so that every
  // LDS address is a per-lane base plus a constant.
  issue(0, 0);
  if (n_tiles > 1) issue(1, 1);
  if (n_tiles > 2) {
    issue(2, 2);
    __builtin_amdgcn_s_waitcnt(10 | (7 << 4) | (15 << 8));   // tile 0 landed, tiles 1-2 may not have
  } else if (n_tiles > 1) {
    wait_vmcnt_5();
  } else {
    wait_vmcnt_0();
  }
  lds_barrier();
  f32x16e scur = scores(0);
  if (TK - 1 > wave_pos0) mask(scur, 0);
  {
    float mx = lane_max(scur);
    rescale_to(half_max(mx) * scale_log2);
  }
  auto step = [&](int t, int buf) {
    // tile t + 1 landed everywhere (tile t + 2 may still load); every wave is past iteration t - 1,
    // so the buffer of tile t - 1 is free for tile t + 3
    if (t + 2 < n_tiles) wait_vmcnt_5(); else wait_vmcnt_0();
    lds_barrier();
    if (t + 3 < n_tiles) issue(t + 3, (buf + 3) & 3);
    f32x16e snext = scores((buf + 1) & 3);
    bf16x8e pb[2];
    float psum = probs(scur, pb);
    if (__any(psum > kRescaleSum)) {   // may move the reference (rare): the exact rule
      const float m_old = m_run;
      rescale_to(half_max(lane_max(scur)) * scale_log2);
      if (m_run != m_old) psum = probs(scur, pb);
    }
    l_run += psum;
    // the 12 MFMAs with their 12 key reads and the 56 VALU operations of the exponentials form one
    // block, left to the scheduler (fixed patterns of 3 or 5 VALU operations per MFMA measured
    // slower). The empty asm keeps the exponentials in this block: without it they sink past the
    // branch below, next to their use in P.V, and nothing runs between the score MFMAs.
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(l_run));
    if ((t + 1) * TK + TK - 1 > wave_pos0 && t + 1 < n_tiles) mask(snext, t + 1);
    pv(buf, pb);
    // the 16 transpose reads first, then the 8 MFMAs: their LDS latency is not waited out one by one
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    scur = snext;
  };
  for (int t = 0; t < n_tiles; t += 4) {
    step(t, 0);
    if (t + 1 >= n_tiles) break;
    step(t + 1, 1);
    if (t + 2 >= n_tiles) break;
    step(t + 2, 2);
    if (t + 3 >= n_tiles) break;
    step(t + 3, 3);
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
  static std::atomic<uint32_t> lds_set{0};
  e = ensure_lds_limit(lds_set, {{(const void*)xp::attn_explicit, xp::LDS_BYTES}});
  if (e != hipSuccess) return e;
  const int n_qb = (n_q + xp::BM - 1) / xp::BM;
  hipLaunchKernelGGL(xp::attn_explicit, dim3(batch * H * n_qb), dim3(256), xp::LDS_BYTES, stream, (const bf16*)q_nope,
                     (const bf16*)q_rope, (const bf16*)cache, seq_off, seq_len, (const bf16*)kc, (const bf16*)vv, H, n_q,
                     max_seq_len, n_qb, L.rope_base, L.softmax_scale * kLog2e, (bf16*)o, lse);
  return hipGetLastError();
}

}  // namespace mla
