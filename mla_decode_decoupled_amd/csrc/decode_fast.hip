// MFMA latent-attention kernel for the DeepSeek-V2/V3 shape: 128 heads, 512-dim latent,
// 64-dim decoupled position part, bf16 storage, fp32 accumulation.
//
// Absorbed, the layer is a multi-query attention whose shared key is the whole 576-wide cached
// row and whose shared value is the first 512 columns of that same row ("旋转约束下的压缩：从 RoPE
// 到 DeepSeek MLA", section "MHA-MQA 切换机制"; "从零理解 MLA", closing figure: the cached latent
// feeds both the score and the value sum). One cache tile in LDS therefore serves 128 heads and
// both contractions.
//
// One workgroup (4 waves) takes one (query row, split chunk) and walks the chunk in tiles of
// 32 keys:
//   * tiles stream HBM -> LDS with direct 16-byte global_load_lds, three buffers, two tiles in
//     flight. The global addresses are permuted so that LDS holds an XOR-swizzled layout
//     (16-byte chunk c of row r sits at c ^ f(r) within its group of 8), which makes both LDS read
//     patterns below bank-conflict free;
//   * scores: wave w owns heads 32w..32w+31 and computes S^T[32 keys x 32 heads] = K Q_w^T with
//     36 MFMA 32x32x16 over the 576 dims; its queries stay in registers for the whole chunk;
//   * softmax per head in log2 units against a fixed reference: m_ref is the head's max over the
//     chunk's first tile and probabilities are 2^(s - m_ref). Softmax is exact for any reference,
//     so the accumulator is never rescaled. Overflow is impossible while every later score stays
//     below m_ref + 64; if one does not, the workgroup leaves the MFMA loop and recomputes its
//     chunk with exact_chunk(), a slow VALU online softmax (correct for any input, never taken
//     on realistic scores). Keys more than 126 below the reference lose weight under 2^-126
//     relative to the first tile's largest key;
//   * P (bf16) goes to LDS; wave w then owns latent columns 128w..128w+127 for all 128 heads and
//     computes O^T += V^T P^T, reading V^T straight from the row-major tile with the gfx950
//     transpose read ds_read_b64_tr_b16. V is read from LDS once per workgroup.
// The chunk result is either final (one chunk: z = O / l, lse) or a split-K partial (O, m, l)
// that attn_merge combines by log-sum-exp.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace fast {

constexpr int H = 128;
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;            // 576 elements
constexpr int ROW_BYTES = ROW * 2;      // 1152
constexpr int ROW_CHUNKS = ROW_BYTES / 16;  // 72 chunks of 16 bytes
constexpr int TILE = 32;                // keys per tile
constexpr int NBUF = 3;
constexpr int TILE_BYTES = TILE * ROW_BYTES;              // 36864
constexpr int TILE_SLOTS = TILE * ROW_CHUNKS;             // 2304 16-byte slots
constexpr int WAVES = 4;
constexpr int SLOTS_PER_WAVE = TILE_SLOTS / WAVES;        // 576
constexpr int DMA_PER_WAVE = SLOTS_PER_WAVE / 64;         // 9 instructions
constexpr int P_STRIDE = 80;            // bytes per head row of P (64 + 16 pad: conflict-free b128 reads)
constexpr float HEADROOM = 64.0f;       // log2 units: P values stay <= 2^64

static_assert(TILE_SLOTS % (WAVES * 64) == 0, "tile must split into whole DMA instructions");
static_assert(ROW_CHUNKS % 8 == 0, "swizzle groups of 8 chunks");

struct Smem {
  unsigned char tile[NBUF][TILE_BYTES];
  unsigned char p[H * P_STRIDE];
  float lsum[H];
  int restart[WAVES];
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
// physical 16-byte chunk of logical chunk c in tile row r (an involution)
__device__ __forceinline__ int phys_chunk(int c, int r) { return (c & ~7) | ((c ^ swz(r)) & 7); }

// Workgroup barrier for LDS traffic only. __syncthreads() carries a workgroup fence, and because
// the tile DMA writes LDS the fence would wait for every DMA in flight (vmcnt(0)), which would
// serialise the prefetch. Each wave instead waits for its own tile DMA explicitly (wait_vmcnt_*)
// and for its own LDS accesses here; the memory clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte-per-lane HBM -> LDS copy: lane l's 16 bytes land at lds_base + 16 * l. Written as
// inline asm so the compiler does not treat later LDS reads of *other* tile buffers as possibly
// aliasing this in-flight write (it would insert vmcnt(0) before them). The instruction has no
// register results; completion is tracked with explicit vmcnt waits. One wait state separates the
// M0 write from the LDS-DMA instruction that reads it.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_vmcnt_9() { __builtin_amdgcn_s_waitcnt((9 & 15) | (7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_vmcnt_0() { __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8)); }

// Exact fallback for one (query row, chunk): per head, a float32 online softmax that rescales
// its running sum and latent accumulator at every block of 256 keys. Same outputs as the MFMA
// path (final z/lse with one chunk, otherwise a partial in log2 units). Kept out of line so the
// MFMA loop's register allocation does not see it.
__device__ __noinline__ void exact_chunk(const bf16* __restrict__ q_packed, const unsigned char* __restrict__ kv,
                                         size_t rh0, int j0, int j1, float scale_log2, int n_chunks, int k,
                                         float* __restrict__ part_acc, float* __restrict__ part_ml,
                                         float* __restrict__ z, float* __restrict__ lse, unsigned char* smem) {
  float* qs = reinterpret_cast<float*>(smem);   // [ROW]
  float* ps = qs + ROW;                         // [256]
  float* red = ps + 256;                        // [8]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int h = 0; h < H; ++h) {
    const size_t rh = rh0 + h;
    for (int d = tid; d < ROW; d += 256) qs[d] = (float)q_packed[rh * ROW + d];
    __syncthreads();
    float m = -INFINITY, l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
    for (int jt = j0; jt < j1; jt += 256) {
      const int j = jt + tid;
      float s = -INFINITY;
      if (j < j1) {
        const bf16* r = reinterpret_cast<const bf16*>(kv + (int64_t)j * ROW_BYTES);
        float dot = 0.0f;
        for (int d = 0; d < ROW; ++d) dot = fmaf(qs[d], (float)r[d], dot);
        s = dot * scale_log2;
      }
      float bm = warp_max(s);
      if (lane == 0) red[w] = bm;
      __syncthreads();
      bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();
      const float m_new = fmaxf(m, bm);
      const float a = exp2f(m - m_new);
      const float p = j < j1 ? exp2f(s - m_new) : 0.0f;
      ps[tid] = p;
      float bs = warp_sum(p);
      if (lane == 0) red[4 + w] = bs;
      __syncthreads();
      l = l * a + (red[4] + red[5] + red[6] + red[7]);
      const int nt = min(256, j1 - jt);
      acc0 *= a;
      acc1 *= a;
      for (int jj = 0; jj < nt; ++jj) {
        const bf16* r = reinterpret_cast<const bf16*>(kv + (int64_t)(jt + jj) * ROW_BYTES);
        acc0 = fmaf(ps[jj], (float)r[tid], acc0);
        acc1 = fmaf(ps[jj], (float)r[tid + 256], acc1);
      }
      m = m_new;
      __syncthreads();
    }
    if (n_chunks == 1) {
      z[rh * DC + tid] = acc0 / l;
      z[rh * DC + tid + 256] = acc1 / l;
      if (lse != nullptr && tid == 0) lse[rh] = (m + log2f(l)) * kLn2;
    } else {
      const size_t slot = rh * n_chunks + k;
      part_acc[slot * DC + tid] = acc0;
      part_acc[slot * DC + tid + 256] = acc1;
      if (tid == 0) {
        part_ml[slot * 2 + 0] = m;
        part_ml[slot * 2 + 1] = l;
      }
    }
  }
}

__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_attn_fast(const bf16* __restrict__ q_packed, const bf16* __restrict__ cache,
                 const int64_t* __restrict__ seq_off, const int32_t* __restrict__ seq_len, int n_q, float scale_log2,
                 int chunk_len, int n_chunks, float* __restrict__ part_acc, float* __restrict__ part_ml,
                 float* __restrict__ z, float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int k = blockIdx.x, bt = blockIdx.y;
  const int b = bt / n_q, t = bt % n_q;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int n_vis = seq_len[b] - n_q + t + 1;
  const int j0 = k * chunk_len;
  const int j1 = min(j0 + chunk_len, n_vis);
  const size_t rh0 = (size_t)bt * H;

  if (j0 >= j1) {  // empty chunk (only possible with several chunks): contributes nothing
    if (threadIdx.x < H) {
      part_ml[((rh0 + threadIdx.x) * n_chunks + k) * 2 + 0] = -INFINITY;
      part_ml[((rh0 + threadIdx.x) * n_chunks + k) * 2 + 1] = 0.0f;
    }
    return;
  }
  const int n_tiles = (j1 - j0 + TILE - 1) / TILE;
  const unsigned char* kv = reinterpret_cast<const unsigned char*>(cache + seq_off[b] * (int64_t)ROW);

  // ---- DMA plan: this lane's 9 slots of every tile (row r, logical chunk c); same for each tile.
  // Slot (row r, physical chunk p) of the LDS tile is filled from logical chunk phys_chunk(p, r)
  // of key r: dma_off = r * ROW_BYTES + 16 * phys_chunk(p, r).
  int dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int it = 0; it < DMA_PER_WAVE; ++it) {
    const int slot = w * SLOTS_PER_WAVE + it * 64 + lane;
    const int r = slot / ROW_CHUNKS, p = slot % ROW_CHUNKS;
    dma_off[it] = r * ROW_BYTES + phys_chunk(p, r) * 16;
  }
  auto issue_tile = [&](int tile) {
    const int key0 = j0 + tile * TILE;
    const unsigned char* src0 = kv + (int64_t)key0 * ROW_BYTES;
    const uint32_t dst = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, sm.tile[tile % NBUF] + (w * SLOTS_PER_WAVE) * 16);
    if (key0 + TILE <= j1) {
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) dma16(src0 + dma_off[it], __builtin_amdgcn_readfirstlane(dst + it * 64 * 16));
    } else {  // tail tile: rows past the end re-read the last valid row (their scores are masked)
      const int last = j1 - 1 - key0;
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) {
        const int r = dma_off[it] / ROW_BYTES;
        const int off = dma_off[it] - (r > last ? r - last : 0) * ROW_BYTES;
        dma16(src0 + off, __builtin_amdgcn_readfirstlane(dst + it * 64 * 16));
      }
    }
  };

  // ---- queries of this wave's 32 heads: B operand fragments of the score MFMA (36 x 8 bf16)
  bf16x8 qf[ROW / 16];
  {
    const bf16* q = q_packed + (rh0 + w * 32 + l32) * ROW + 8 * g;
#pragma unroll
    for (int s = 0; s < ROW / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(q + 16 * s);
  }
  wait_vmcnt_0();   // queries resident before the loop, so no wait for them lands inside it

  if (threadIdx.x < WAVES) sm.restart[threadIdx.x] = 0;
  bool overflowed = false;
  issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  // O^T accumulators: [col block cb][head block hb], 16 fp32 each
  f32x16 oacc[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][hb][r] = 0.0f;

  float m_ref = -INFINITY;  // per lane: head 32w + l32 (both lane halves agree); set by the first tile
  float l_run = 0.0f;       // per lane: sum over this lane's half of the keys

  // per-lane LDS byte offsets
  // scores: A operand row = key l32, logical chunk 2s + g -> phys (s/4)*8 + ((2(s%4)+g) ^ swz(l32))
  int qk_off[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) qk_off[s4] = l32 * ROW_BYTES + (((2 * s4 + g) ^ swz(l32)) & 7) * 16;
  // values: transpose reads. lane = 16q + L; row = 16s + 8g + 4h + L/4; col = 128w + 32cb + 16(q&1) + 4(L&3)
  const int q16 = lane >> 4, L = lane & 15;
  int pv_off[2][2];  // [cb & 1][h]
#pragma unroll
  for (int cbo = 0; cbo < 2; ++cbo)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g + 4 * h + (L >> 2);
      const int clow = 4 * cbo + 2 * (q16 & 1) + ((L >> 1) & 1);  // logical chunk & 7
      const int ph = (clow ^ (((L >> 2) << 1) | h)) & 7;
      pv_off[cbo][h] = row * ROW_BYTES + (16 * w) * 16 + ph * 16 + (L & 1) * 8;
    }
  const int p_wr = (w * 32 + l32) * P_STRIDE + 4 * g * 2;      // + 16 * j for key block j
  const int p_rd = l32 * P_STRIDE + 8 * g * 2;                  // + hb*32*P_STRIDE + 32*s

  for (int tile = 0; tile < n_tiles; ++tile) {
    if (tile + 1 < n_tiles) wait_vmcnt_9(); else wait_vmcnt_0();
    lds_barrier();  // tile visible to all waves; everyone finished the previous tile's PV
    if (tile + 2 < n_tiles) issue_tile(tile + 2);

    const unsigned char* tb = sm.tile[tile % NBUF];
    // ---------------- scores S^T = K Q^T for this wave's heads
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < ROW / 16; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(tb + qk_off[s & 3] + (s >> 2) * 128);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
    }
    // ---------------- online softmax (lane: head 32w + l32, keys 8j + 4g + i of the tile)
    const int key0 = j0 + tile * TILE;
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * g + (r & 3);
      const float s = (key0 + kk < j1) ? sacc[r] * scale_log2 : -INFINITY;
      sacc[r] = s;
      tmax = fmaxf(tmax, s);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (m_ref == -INFINITY) m_ref = tmax;  // first tile of the chunk fixes the reference
    const bool overflow_risk = tmax > m_ref + HEADROOM;
    if (__any(overflow_risk) && lane == 0) sm.restart[w] = 1;
    float psum = 0.0f;
    unsigned short pb16[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f(sacc[r] - m_ref);
      psum += p;
      pb16[r] = __builtin_bit_cast(unsigned short, (bf16)p);
    }
    l_run += psum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 v = make_uint2((uint32_t)pb16[4 * j] | ((uint32_t)pb16[4 * j + 1] << 16),
                                 (uint32_t)pb16[4 * j + 2] | ((uint32_t)pb16[4 * j + 3] << 16));
      *reinterpret_cast<uint2*>(sm.p + p_wr + 16 * j) = v;
    }
    lds_barrier();  // P and rescale factors of all heads visible

    // ---------------- a score far above the reference: leave for the exact path (see header)
    if (__builtin_amdgcn_readfirstlane(sm.restart[0] | sm.restart[1] | sm.restart[2] | sm.restart[3]) != 0) {
      overflowed = true;
      break;
    }
    // ---------------- O^T += V^T P^T for this wave's 128 latent columns, all heads
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 pf[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        pf[hb] = *reinterpret_cast<const bf16x8*>(sm.p + p_rd + hb * 32 * P_STRIDE + 32 * s);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const unsigned char* base = tb + s * 16 * ROW_BYTES + (cb >> 1) * 128;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MLA_LDS(i16x4, base + pv_off[cb & 1][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(MLA_LDS(i16x4, base + pv_off[cb & 1][1]));
        bf16x8 af;
        const bf16x4 lo16 = __builtin_bit_cast(bf16x4, lo), hi16 = __builtin_bit_cast(bf16x4, hi);
        af[0] = lo16[0]; af[1] = lo16[1]; af[2] = lo16[2]; af[3] = lo16[3];
        af[4] = hi16[0]; af[5] = hi16[1]; af[6] = hi16[2]; af[7] = hi16[3];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          oacc[cb][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[hb], oacc[cb][hb], 0, 0, 0);
      }
    }
  }

  if (overflowed) {
    wait_vmcnt_0();   // no DMA may still target LDS
    lds_barrier();
    exact_chunk(q_packed, kv, rh0, j0, j1, scale_log2, n_chunks, k, part_acc, part_ml, z, lse, smem_raw);
    return;
  }
  // ---- per-head totals: combine the two key halves, publish for every wave
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    sm.lsum[w * 32 + l32] = l_run;
  }
  lds_barrier();
  if (n_chunks == 1) {
    if (lse != nullptr && g == 0) lse[rh0 + w * 32 + l32] = (m_ref + log2f(l_run)) * kLn2;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = hb * 32 + l32;
      const float inv = 1.0f / sm.lsum[head];
      float* dst = z + (rh0 + head) * DC + 128 * w + 4 * g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v = {oacc[cb][hb][4 * j] * inv, oacc[cb][hb][4 * j + 1] * inv, oacc[cb][hb][4 * j + 2] * inv,
                     oacc[cb][hb][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * j) = v;
        }
    }
  } else {
    if (g == 0) {
      float* ml = part_ml + ((rh0 + w * 32 + l32) * n_chunks + k) * 2;
      ml[0] = m_ref;
      ml[1] = l_run;
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = hb * 32 + l32;
      float* dst = part_acc + ((rh0 + head) * n_chunks + k) * (size_t)DC + 128 * w + 4 * g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v = {oacc[cb][hb][4 * j], oacc[cb][hb][4 * j + 1], oacc[cb][hb][4 * j + 2], oacc[cb][hb][4 * j + 3]};
          *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * j) = v;
        }
    }
  }
}

}  // namespace fast

bool attn_fast_supported(const LayerDims& L) {
  return L.n_heads == fast::H && L.d_latent == fast::DC && L.d_rope == fast::DR;
}

hipError_t launch_attn_fast(const LayerDims& L, int batch, int n_q, const void* q_packed, const void* cache,
                            const int64_t* seq_off, const int32_t* seq_len, const SplitPlan& plan, void* workspace,
                            float* z, float* lse, hipStream_t stream) {
  float* part_acc = (float*)workspace;
  float* part_ml = plan.n_chunks > 1 ? part_acc + (size_t)batch * n_q * fast::H * plan.n_chunks * fast::DC : nullptr;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)fast::decode_attn_fast, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(fast::Smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(plan.n_chunks, batch * n_q);
  hipLaunchKernelGGL(fast::decode_attn_fast, grid, dim3(256), sizeof(fast::Smem), stream, (const bf16*)q_packed,
                     (const bf16*)cache, seq_off, seq_len, n_q, L.softmax_scale * kLog2e, plan.chunk_len,
                     plan.n_chunks, part_acc, part_ml, z, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_chunks == 1) return e;
  return launch_attn_merge(batch * n_q * fast::H, plan.n_chunks, fast::DC, part_acc, part_ml, z, lse, stream);
}

}  // namespace mla
