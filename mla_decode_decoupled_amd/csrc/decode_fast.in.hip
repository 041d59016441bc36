@GENERATED_NOTE@
// MFMA latent-attention kernel for the DeepSeek-V2/V3 shape: 128 heads, 512-dim latent,
// 64-dim decoupled position part, bf16 storage, fp32 accumulation.
//
// Absorbed, the layer is a multi-query attention whose shared key is the whole 576-wide cached
// row and whose shared value is the first 512 columns of that same row ("旋转约束下的压缩：从 RoPE
// 到 DeepSeek MLA", section "MHA-MQA 切换机制"; "从零理解 MLA", closing figure: the cached latent
// feeds both the score and the value sum). One cache tile in LDS therefore serves 128 heads and
// both contractions.
//
// One workgroup (4 waves, one per SIMD) takes one (query row, split chunk) and walks the chunk
// in tiles of 32 keys:
//   * tiles stream HBM -> LDS with direct 16-byte global_load_lds, three buffers, two tiles in
//     flight. The global addresses are permuted so that LDS holds an XOR-swizzled layout
//     (16-byte chunk c of row r sits at c ^ f(r) within its group of 8), which makes both LDS read
//     patterns below bank-conflict free;
//   * scores: wave w owns heads 32w..32w+31 and computes S^T[32 keys x 32 heads] = K Q_w^T with
//     36 chained MFMA 32x32x16 over the 576 dims. The latent part of its queries stays in VGPRs
//     for the whole chunk, the 64-dim position part is read from LDS;
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
// The loop is software-pipelined with one barrier per tile: iteration t computes the scores of
// tile t+1, then runs the P.V MFMAs of tile t with the softmax VALU work of tile t+1 interleaved
// between them (P is double-buffered in LDS), so the exponentials hide under the MFMAs.
// The chunk result is either final (one chunk: z = O / l, lse) or a split-K partial (O, m, l)
// that attn_merge combines by log-sum-exp.
//
// Register plan (per lane, 512 = 256 VGPRs + 256 AGPRs with one wave per SIMD):
//   a[0:255]    O^T accumulator, 16 blocks of 32x32 fp32 (asm operands constrained to AGPRs)
//   v[128:255]  latent queries, 32 MFMA B fragments (pinned by physical-register constraints)
//   v[112:127]  score accumulator S^T; v[80:111] operand rings of the two MFMA phases
//   v[0:79]     everything the compiler allocates (addresses, softmax, DMA offsets)
// The two MFMA phases are inline asm because at this occupancy the compiler's allocator spills
// whatever split it picks. Hazards it cannot see inside asm are handled explicitly: LDS operands
// are waited for with lgkmcnt in issue order, chained MFMAs use exactly the same accumulator (no
// wait states needed), an operand ring slot is only rewritten after the MFMA reading it has
// issued, and 20 wait states separate the last score MFMA from VALU reads of its result.
#include <cstddef>

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
constexpr int QR_STRIDE = 144;          // bytes per head row of the position queries (128 + 16 pad)
constexpr float HEADROOM = 64.0f;       // log2 units: P values stay <= 2^64
constexpr int QS_STRIDE = 1024 + 16;    // bytes per staged query row (latent part + pad)
constexpr int ES_STRIDE = 512 + 4;      // floats per staged output row (+ pad)

static_assert(TILE_SLOTS % (WAVES * 64) == 0, "tile must split into whole DMA instructions");
static_assert(ROW_CHUNKS % 8 == 0, "swizzle groups of 8 chunks");

struct Smem {
  unsigned char tile[NBUF][TILE_BYTES];
  unsigned char p[2][H * P_STRIDE];     // double-buffered: tile t read while tile t+1 is written
  unsigned char qrope[H * QR_STRIDE];
  float lsum[H];
  int restart[WAVES];
};
// Query staging (before the loop) and output staging (after it) reuse tiles, P and the position
// queries; both stop short of lsum, which the epilogue still reads.
static_assert(H * QS_STRIDE <= offsetof(Smem, lsum), "query staging must end before lsum");
static_assert(64 * ES_STRIDE * 4 <= offsetof(Smem, lsum), "output staging must end before lsum");

typedef int v16i __attribute__((vector_size(64)));

// LDS has 64 banks of 4 bytes and serves 16 lanes of a 16-byte read per cycle. A cache row is
// 1152 bytes (= 128 mod 256), so rows of equal parity share bank offsets; swz() is injective on
// the even and on the odd rows of any 16 consecutive rows (score reads: 16 rows, same chunk), and
// rows r, r+2 of an aligned group of 4 differ in bit 2 (transpose reads: 4 rows x 4 chunks).
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
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
// Nothing else in this kernel uses M0 (the compiler warns that it does not track a clobber of
// that reserved register, so this must stay true).
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

  // ---- DMA plan: slot (row r, physical chunk p) of the LDS tile is filled from logical chunk
  // phys_chunk(p, r) of key r: dma_off = r * ROW_BYTES + 16 * phys_chunk(p, r).
  uint32_t dma_off[DMA_PER_WAVE];
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
    if (key0 + TILE <= j1) {  // full tile: SGPR base + 32-bit lane offsets, no VALU work
      const uint64_t sb = (uint64_t)(uintptr_t)src0;
      const uint64_t sbase = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
      const uint32_t sdst = __builtin_amdgcn_readfirstlane(dst);
      asm volatile(
@DMA_ASM@
          ::[b] "s"(sbase), [m] "s"(sdst), [o0] "v"(dma_off[0]), [o1] "v"(dma_off[1]), [o2] "v"(dma_off[2]),
          [o3] "v"(dma_off[3]), [o4] "v"(dma_off[4]), [o5] "v"(dma_off[5]), [o6] "v"(dma_off[6]),
          [o7] "v"(dma_off[7]), [o8] "v"(dma_off[8])
          : "memory", "m0");
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

  // ---- queries of this wave's 32 heads (32w .. 32w+31).
  // Latent part: 32 B fragments (8 bf16 per lane: dims 16s + 8g .. +7 of head 32w + l32) for
  // v[128:255]. Loaded straight from global memory, every instruction would touch 32 rows 1152 B
  // apart, so the rows are staged through LDS instead: each wave copies its 32 rows with 1 KB
  // direct global->LDS loads (8 whole cache lines each) into slots QS_STRIDE bytes apart (the
  // 16-byte pad puts the 16 heads of one LDS phase on 16 different bank groups), then reads its
  // fragments. The staging area is the first tile buffers, free until the first tile DMA.
  // Position part: 4 fragments per lane, kept in LDS and read by every score phase.
  const int qhead = w * 32 + l32;
  const bf16* qrow = q_packed + (rh0 + qhead) * ROW + 8 * g;
  const uint32_t qstage = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, &sm.tile[0][0]) + w * 32 * QS_STRIDE;
  {
    const unsigned char* qw = reinterpret_cast<const unsigned char*>(q_packed + (rh0 + w * 32) * ROW) + 16 * lane;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) dma16(qw + i * ROW_BYTES, __builtin_amdgcn_readfirstlane(qstage + i * QS_STRIDE));
  }
  bf16x8 qr_frag[DR / 16];
#pragma unroll
  for (int s = 0; s < DR / 16; ++s) qr_frag[s] = *reinterpret_cast<const bf16x8*>(qrow + DC + 16 * s);
  wait_vmcnt_0();   // the staged rows and the position fragments are in
  v16i q0, q1, q2, q3, q4, q5, q6, q7;
  asm volatile(
@QLOAD_ASM@
      : "=&{v[128:143]}"(q0), "=&{v[144:159]}"(q1), "=&{v[160:175]}"(q2), "=&{v[176:191]}"(q3),
        "=&{v[192:207]}"(q4), "=&{v[208:223]}"(q5), "=&{v[224:239]}"(q6), "=&{v[240:255]}"(q7)
      : [a] "v"(qstage + l32 * QS_STRIDE + 16 * g)
      : "memory");
  lds_barrier();   // every wave holds its fragments: the staging area is free for the tiles
#pragma unroll
  for (int s = 0; s < DR / 16; ++s)
    *reinterpret_cast<bf16x8*>(sm.qrope + qhead * QR_STRIDE + (2 * s + g) * 16) = qr_frag[s];

  bool ovf = false;   // this wave saw a score far above its reference (uniform)

  // O^T accumulators: [col block cb][head block hb], 16 fp32 each, zeroed in AGPRs by MFMAs of
  // zero operands (a plain zero initialisation would be built in VGPRs first and copied over)
  f32x16 o00, o01, o02, o03, o10, o11, o12, o13, o20, o21, o22, o23, o30, o31, o32, o33;
  {
    const bf16x8 zf = {};
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %1, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %3, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %4, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %5, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %6, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %7, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %8, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %9, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %10, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %11, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %12, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %13, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %14, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %15, %[z], %[z], 0"
        : "=a"(o00), "=a"(o01), "=a"(o02), "=a"(o03), "=a"(o10), "=a"(o11), "=a"(o12), "=a"(o13),
          "=a"(o20), "=a"(o21), "=a"(o22), "=a"(o23), "=a"(o30), "=a"(o31), "=a"(o32), "=a"(o33)
        : [z] "v"(zf));
  }

  float m_ref = -INFINITY;  // per lane: head 32w + l32 (both lane halves agree); set by the first tile
  float l_run = 0.0f;       // per lane: sum over this lane's half of the keys

  // per-lane LDS byte offsets
  // scores: A operand row = key l32, logical chunk 2s + g -> phys (s/4)*8 + ((2(s%4)+g) ^ swz(l32))
  uint32_t qk_off[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) qk_off[s4] = l32 * ROW_BYTES + (((2 * s4 + g) ^ swz(l32)) & 7) * 16;
  const uint32_t qr_addr = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, sm.qrope + qhead * QR_STRIDE + 16 * g);
  // values: transpose reads. lane = 16q + L; row = 16s + 8g + 4h + L/4; col = 128w + 32cb + 16(q&1) + 4(L&3)
  const int q16 = lane >> 4, L = lane & 15;
  uint32_t pv_off[2][2];  // [cb & 1][h]
#pragma unroll
  for (int cbo = 0; cbo < 2; ++cbo)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g + 4 * h + (L >> 2);
      const int clow = 4 * cbo + 2 * (q16 & 1) + ((L >> 1) & 1);  // logical chunk & 7
      const int ph = (clow ^ swz(row)) & 7;
      pv_off[cbo][h] = row * ROW_BYTES + (16 * w) * 16 + ph * 16 + (L & 1) * 8;
    }
  const uint32_t p_base = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, &sm.p[0][0]);
  const uint32_t p_wr = p_base + (w * 32 + l32) * P_STRIDE + 4 * g * 2;   // + 16 * j for key block j
  const uint32_t p_rd = p_base + l32 * P_STRIDE + 8 * g * 2;
  constexpr uint32_t P_BUF = H * P_STRIDE;

  auto tile_lds = [&](int tile) { return (uint32_t)(uintptr_t)MLA_LDS(unsigned char, sm.tile[tile % NBUF]); };

  // Scores of one tile into v[112:127]. The same asm block issues the DMA of the tile after it
  // (9 global_load_lds spread between the MFMAs, so the VMEM issue overlaps the matrix work).
  // That tile's buffer held tile - 2, which every wave finished reading before the barrier that
  // opened this iteration. With no tile left to load, the DMA reads this query row's packed
  // queries (valid memory of H * ROW_BYTES bytes) into that buffer, which is not read again.
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(q_packed + rh0 * ROW);
  auto scores = [&](int tile, f32x16& sacc) {
    const uint32_t tb = tile_lds(tile);
    const int dt = tile + 1;
    const int key0 = j0 + dt * TILE;
    const unsigned char* src = dt < n_tiles ? kv + (int64_t)key0 * ROW_BYTES : qbytes;
    uint32_t o[DMA_PER_WAVE];
#pragma unroll
    for (int it = 0; it < DMA_PER_WAVE; ++it) o[it] = dma_off[it];
    if (dt < n_tiles && key0 + TILE > j1) {  // tail tile: rows past the end re-read the last valid row
      const int last = j1 - 1 - key0;
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) {
        const int r = dma_off[it] / ROW_BYTES;
        o[it] = dma_off[it] - (r > last ? r - last : 0) * ROW_BYTES;
      }
    }
    const uint64_t sb = (uint64_t)(uintptr_t)src;
    const uint64_t sbase = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
    const uint32_t sdst = __builtin_amdgcn_readfirstlane(tile_lds(dt) + (w * SLOTS_PER_WAVE) * 16);
    asm volatile(
@QK_ASM@
        : "=&{v[112:127]}"(sacc)
        : [k0] "v"(tb + qk_off[0]), [k1] "v"(tb + qk_off[1]), [k2] "v"(tb + qk_off[2]), [k3] "v"(tb + qk_off[3]),
          [qr] "v"(qr_addr), "{v[128:143]}"(q0), "{v[144:159]}"(q1), "{v[160:175]}"(q2), "{v[176:191]}"(q3),
          "{v[192:207]}"(q4), "{v[208:223]}"(q5), "{v[224:239]}"(q6), "{v[240:255]}"(q7),
          [b] "s"(sbase), [m] "s"(sdst), [o0] "v"(o[0]), [o1] "v"(o[1]), [o2] "v"(o[2]), [o3] "v"(o[3]),
          [o4] "v"(o[4]), [o5] "v"(o[5]), [o6] "v"(o[6]), [o7] "v"(o[7]), [o8] "v"(o[8])
        : "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87", "v88", "v89", "v90", "v91", "v92", "v93", "v94",
          "v95", "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108",
          "v109", "v110", "v111", "memory", "m0");
  };

  // softmax of one tile in C++ (first tile: fixes the reference; partial tail tile: masks keys
  // past the end). Writes the tile's P buffer and flags a score far above the reference.
  auto softmax_masked = [&](int tile, f32x16 sacc) {
    const int key0 = j0 + tile * TILE;
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * g + (r & 3);
      const float sv = (key0 + kk < j1) ? sacc[r] * scale_log2 : -INFINITY;
      sacc[r] = sv;
      tmax = fmaxf(tmax, sv);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (m_ref == -INFINITY) m_ref = tmax;
    ovf |= __any(tmax > m_ref + HEADROOM);
    float psum = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2f(sacc[r] - m_ref), p1 = exp2f(sacc[r + 1] - m_ref);
      psum += p0 + p1;
      pk[r / 2] = (uint32_t)__builtin_bit_cast(unsigned short, (bf16)p0) |
                  ((uint32_t)__builtin_bit_cast(unsigned short, (bf16)p1) << 16);
    }
    l_run += psum;
    unsigned char* pw = &sm.p[tile & 1][0] + (w * 32 + l32) * P_STRIDE + 4 * g * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint2*>(pw + 16 * j) = make_uint2(pk[2 * j], pk[2 * j + 1]);
  };

  // P.V of tile t with the softmax of the full tile t+1 (scores in v[112:127]) interleaved
  auto pv_softmax = [&](int tile, f32x16& sacc) {
    const uint32_t tb = tile_lds(tile);
    float mx;
    asm volatile(
@PVSM_ASM@
        : [o00] "+a"(o00), [o01] "+a"(o01), [o02] "+a"(o02), [o03] "+a"(o03), [o10] "+a"(o10), [o11] "+a"(o11),
          [o12] "+a"(o12), [o13] "+a"(o13), [o20] "+a"(o20), [o21] "+a"(o21), [o22] "+a"(o22), [o23] "+a"(o23),
          [o30] "+a"(o30), [o31] "+a"(o31), [o32] "+a"(o32), [o33] "+a"(o33), [l] "+v"(l_run), [mx] "=&v"(mx),
          "+{v[112:127]}"(sacc)
        : [p] "v"(p_rd + (tile & 1) * P_BUF), [v00] "v"(tb + pv_off[0][0]), [v01] "v"(tb + pv_off[0][1]),
          [v10] "v"(tb + pv_off[1][0]), [v11] "v"(tb + pv_off[1][1]), [sc] "s"(scale_log2), [nm] "v"(-m_ref),
          [pw] "v"(p_wr + ((tile + 1) & 1) * P_BUF)
        : "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87", "v88", "v89", "v90", "v91", "v92", "v93", "v94",
          "v95", "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108",
          "v109", "v110", "v111", "memory");
    ovf |= __any(mx * scale_log2 > m_ref + HEADROOM);
  };

  // ---- the loop. Iteration t >= 0: P.V of tile t fused with the softmax of tile t+1 (its scores
  // computed just before); iteration -1 only scores tile 0 and fixes the reference in C++.
  // Exactly one site per asm phase keeps the register assignment simple for the compiler.
  issue_tile(0);
  for (int tile = -1; tile < n_tiles; ++tile) {
    wait_vmcnt_0();   // tile t+1 (the only DMA in flight) landed
    lds_barrier();    // P(t) and tile t+1 visible to all waves; iteration t-1 finished everywhere
    f32x16 sacc;
    if (tile + 1 < n_tiles) scores(tile + 1, sacc);
    if (tile < 0) {
      softmax_masked(0, sacc);
      continue;
    }
    if (tile + 1 >= n_tiles) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = -INFINITY;   // no next tile: the fused softmax adds 0
    } else if (j0 + (tile + 2) * TILE > j1) {               // partial next tile: mask keys past the end
      const int key0 = j0 + (tile + 1) * TILE;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + 4 * g + (r & 3) >= j1) sacc[r] = -INFINITY;
    }
    pv_softmax(tile, sacc);
  }

  // A score far above the reference makes later probabilities overflow (inf / NaN in the
  // accumulator, harmless to the hardware); the loop still runs to its end, and the chunk is then
  // recomputed by the exact path. The flags meet in LDS once, after the loop.
  if (lane == 0) sm.restart[w] = ovf ? 1 : 0;
  __syncthreads();
  const bool overflowed = (sm.restart[0] | sm.restart[1] | sm.restart[2] | sm.restart[3]) != 0;
  if (overflowed) {
    wait_vmcnt_0();   // no DMA may still target LDS
    __syncthreads();
    exact_chunk(q_packed, kv, rh0, j0, j1, scale_log2, n_chunks, k, part_acc, part_ml, z, lse, smem_raw);
    return;
  }
  // the accumulator is read by VALU below: 20 wait states after the last MFMA
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(o00), "+a"(o01), "+a"(o02), "+a"(o03), "+a"(o10), "+a"(o11), "+a"(o12), "+a"(o13),
                 "+a"(o20), "+a"(o21), "+a"(o22), "+a"(o23), "+a"(o30), "+a"(o31), "+a"(o32), "+a"(o33));

  // ---- per-head totals: combine the two key halves, publish for every wave
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) sm.lsum[w * 32 + l32] = l_run;
  if (g == 0) {
    if (n_chunks == 1) {
      if (lse != nullptr) lse[rh0 + w * 32 + l32] = (m_ref + log2f(l_run)) * kLn2;
    } else {
      float* ml = part_ml + ((rh0 + w * 32 + l32) * n_chunks + k) * 2;
      ml[0] = m_ref;
      ml[1] = l_run;
    }
  }

  // ---- O^T out through LDS, 64 heads per round. Written straight from the accumulator layout,
  // every store would touch 32 rows; staged, each wave writes whole 2 KB rows (one chunk's
  // partial, or z = O / l when the chunk is the whole sequence) with contiguous 1 KB stores.
  float* stage = reinterpret_cast<float*>(smem_raw);   // [64][ES_STRIDE]
  const f32x16* oacc[4][4] = {{&o00, &o01, &o02, &o03}, {&o10, &o11, &o12, &o13},
                              {&o20, &o21, &o22, &o23}, {&o30, &o31, &o32, &o33}};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();   // the loop (or the previous round's reads) finished everywhere; lsum visible
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float* row = stage + (hh * 32 + l32) * ES_STRIDE + 128 * w + 4 * g;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& o = *oacc[cb][2 * half + hh];
          *reinterpret_cast<f32x4*>(row + 32 * cb + 8 * j) = f32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        }
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int hl = 16 * w + i;
      const size_t head = (size_t)(64 * half + hl);
      f32x4 va = *reinterpret_cast<const f32x4*>(stage + hl * ES_STRIDE + 4 * lane);
      f32x4 vb = *reinterpret_cast<const f32x4*>(stage + hl * ES_STRIDE + 256 + 4 * lane);
      float* dst;
      if (n_chunks == 1) {
        const float inv = 1.0f / sm.lsum[head];
        va *= inv;
        vb *= inv;
        dst = z + (rh0 + head) * DC;
      } else {
        dst = part_acc + ((rh0 + head) * n_chunks + k) * (size_t)DC;
      }
      *reinterpret_cast<f32x4*>(dst + 4 * lane) = va;
      *reinterpret_cast<f32x4*>(dst + 256 + 4 * lane) = vb;
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
