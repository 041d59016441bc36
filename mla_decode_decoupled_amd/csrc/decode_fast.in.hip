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
// in tiles of 32 keys. Wave w scores heads 32w..32w+31 and accumulates latent columns
// 128w..128w+127 of all 128 heads:
//   * tiles stream HBM -> LDS with direct 16-byte global_load_lds into four buffers, two tiles in
//     flight while two are being computed on. The global addresses are permuted so that LDS holds
//     an XOR-swizzled layout (16-byte chunk c of row r sits at c ^ f(r) within its group of 8),
//     which makes both LDS read patterns below bank-conflict free;
//   * scores: S^T[32 keys x 32 heads] = K Q_w^T with 36 chained MFMA 32x32x16 over the 576 dims.
//     The latent part of the wave's queries stays in VGPRs for the whole chunk, the 64-dim
//     position part is read from LDS. The key rows of the A operand are taken in the order pi
//     (below), so that each lane's 16 score registers are exactly the keys its P.V operand needs;
//   * softmax per head in log2 units against a fixed reference: m_ref is the head's max over the
//     chunk's first tile and probabilities are 2^(s - m_ref). Softmax is exact for any reference,
//     so the accumulator is never rescaled. A score above m_ref + 64 makes its probability, and
//     so the lane's running sum of probabilities, exceed 2^64; a sum above that after the loop
//     sets a flag, and the workgroup then recomputes its chunk with exact_chunk(), a slow VALU
//     online softmax (correct for any input, never taken on realistic scores). Keys more than 126
//     below the reference lose weight under 2^-126 relative to the first tile's largest key;
//   * P (bf16) goes through LDS: each wave stores the B fragments of its 32 heads (2 KB) into one
//     of two P buffers, and every wave reads all four head blocks' fragments back. Then
//     O^T[128 columns x 128 heads] += V^T P^T with 32 MFMAs per wave: V^T is read from the
//     row-major tile with the gfx950 transpose read ds_read_b64_tr_b16, and each V^T fragment
//     feeds the four head blocks' MFMAs (each P fragment the four column blocks'), so a wave reads
//     16 KB of operands from LDS per tile for P.V instead of the 32 KB of V^T that all 512 columns
//     of its own heads would take.
// The loop is software-pipelined with one barrier per tile (the tile and P buffers are shared):
// iteration t computes the scores of tile t+1 (and issues the DMA of tile t+3), then runs the
// P.V MFMAs of tile t with the softmax VALU work of tile t+1 interleaved between them, so the
// exponentials hide under the MFMAs, and stores P of tile t+1 for the next iteration. The chunk
// result is either final (one chunk: z = O / l, lse) or a split-K partial (O, m, l) that
// attn_merge_frag combines by log-sum-exp.
//
// Register plan (per lane, 512 = 256 VGPRs + 256 AGPRs with one wave per SIMD):
//   a[0:255]    O^T accumulator, 16 blocks (4 column blocks x 4 head blocks) of 32 latent
//               columns x 32 heads, fp32
//   v[128:255]  latent queries, 32 MFMA B fragments (pinned by physical-register constraints)
//   v[112:127]  score accumulator S^T, softmax in place, then P packed in place (v[112:119])
//   v[64:79]    position part of the queries (4 MFMA B fragments)
//   v[80:111]   operand slots of the two MFMA phases (the score phase uses v[88:111])
//   v[0:79]     everything the compiler allocates (addresses, softmax state, DMA offsets)
// The two MFMA phases are inline asm because at this occupancy the compiler's allocator spills
// whatever split it picks. Hazards it cannot see inside asm are handled explicitly: LDS operands
// are waited for with lgkmcnt in issue order, chained MFMAs use exactly the same accumulator (no
// wait states needed), an operand register is only rewritten after the MFMA reading it has
// issued (plus wait states where a VALU op rewrites it), and 20 wait states separate the last
// score MFMA from VALU reads of its result.
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
constexpr int NBUF = 4;                 // tile buffers: two being computed on, two in flight
constexpr int TILE_BYTES = TILE * ROW_BYTES;              // 36864
constexpr int TILE_SLOTS = TILE * ROW_CHUNKS;             // 2304 16-byte slots
constexpr int WAVES = 4;
constexpr int SLOTS_PER_WAVE = TILE_SLOTS / WAVES;        // 576
constexpr int DMA_PER_WAVE = SLOTS_PER_WAVE / 64;         // 9 instructions
constexpr float HEADROOM = 64.0f;       // log2 units: P values stay <= 2^64
constexpr float kSumLimit = 0x1p64f;    // 2^HEADROOM: a probability sum above it may hide one above it
constexpr int QS_STRIDE = 1024 + 16;    // bytes per staged query row (latent part + pad)
constexpr int ES_STRIDE = 128 + 4;      // floats per staged output row slice (+ pad)

static_assert(TILE_SLOTS % (WAVES * 64) == 0, "tile must split into whole DMA instructions");
static_assert(ROW_CHUNKS % 8 == 0, "swizzle groups of 8 chunks");

// LDS (160 KB): four tile buffers (144 KB), then two P buffers, each P of one tile for all 128
// heads, [head block][key step][lane][8 bf16] (8 KB), written by the wave that scored the head
// block and read by every wave. The query staging before the loop and the output staging after
// it reuse the tile buffers; the overflow flags, the chunk plan and the output's per-head sums sit
// in the last kilobyte of the tile area, clear of both stagings. (The 64-dim position part of the
// queries stays in VGPRs, v[64:79].)
constexpr int PBUF_BYTES = 4 * 2 * 64 * 16;
struct Smem {
  unsigned char tile[NBUF][TILE_BYTES];
  unsigned char pbuf[2][PBUF_BYTES];
};
// The tile DMA sets M0 once per four 1 KB instructions and steps the LDS address with the
// instruction's offset field (0, 1024, 2048, 3072), which moves the global address by the same
// amount: the per-lane global offsets are biased by -1024 (it % 4), plus DMA_BIAS (taken off the
// base pointer). The offset is an unsigned 32-bit VGPR, so it must stay non-negative for every
// row it can name, row 0 included (the re-read rows of a chunk shorter than one tile all name its
// last row, possibly row 0): row * ROW_BYTES + 16 chunk >= 0 and DMA_BIAS >= 3072 make it at least
// DMA_BIAS - 3072.
constexpr int DMA_BIAS = 4096;
static_assert(DMA_BIAS >= 3 * 1024, "DMA offsets must stay non-negative for row 0, instruction offset 3072");
constexpr int FLAGS_OFF = NBUF * TILE_BYTES - 1024;
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(H * QS_STRIDE <= FLAGS_OFF, "query staging must end before the flags");
static_assert(H * ES_STRIDE * 4 <= FLAGS_OFF, "output staging must end before the flags");
constexpr int LSUM_OFF = FLAGS_OFF + 256;   // per-head sums for z = O / l, after the flags and the plan
static_assert(LSUM_OFF + H * 4 <= NBUF * TILE_BYTES, "per-head sums must stay in the tile area");

typedef int v16i __attribute__((vector_size(64)));
typedef int v8i __attribute__((vector_size(32)));

// LDS has 64 banks of 4 bytes and serves 16 lanes of a 16-byte read per cycle. A cache row is
// 1152 bytes (= 128 mod 256), so rows of equal parity share bank offsets; swz() is injective on
// the even and on the odd rows of any 16 consecutive rows (score reads: 16 rows, same chunk), and
// rows r, r+2 of an aligned group of 4 differ in bit 2 (transpose reads: 4 rows x 4 chunks).
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
// physical 16-byte chunk of logical chunk c in tile row r (an involution)
__device__ __forceinline__ int phys_chunk(int c, int r) { return (c & ~7) | ((c ^ swz(r)) & 7); }
// Key order of the score operand: A row r = 8j + 4h + i holds key pi(r) = 16(j/2) + 8h + 4(j%2) + i.
// The MFMA result then gives the lane of key half h the 16 keys 8h..8h+7 and 16+8h..16+8h+7,
// which are its B fragments of the two 16-key steps of P.V. pi maps rows 0-15 and 16-31 onto
// themselves, so the bank pattern of the score reads does not change.
__device__ __forceinline__ int key_of_row(int r) {
  const int j = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + i;
}
// key held in score register rr (0..15) by a lane of key half g
__device__ __forceinline__ int key_of_reg(int rr, int g) { return key_of_row(8 * (rr >> 2) + 4 * g + (rr & 3)); }

// Workgroup barrier for LDS traffic only. __syncthreads() carries a workgroup fence, and because
// the tile DMA writes LDS the fence would wait for every DMA in flight (vmcnt(0)), which would
// serialise the prefetch. Each wave instead waits for its own tile DMA explicitly (wait_vmcnt_*)
// and for its own LDS accesses here; the memory clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Phase stamps, compiled only into the diagnostic build (-DMLA_PHASE_STAMPS, libmla_stamps.so):
// thread 0 of each workgroup records the shader clock counter (s_memtime) at the phase boundaries
// of the attention kernels, the 100 MHz counter (s_memrealtime) at entry and exit, and what its
// chunk was. Slots: 0 entry, 1 chunk known, 2 queries in registers (128-head kernel), 3 first tiles
// issued (head-split kernel: queries and first tiles landed), 4 loop done, 5 exit with every store
// completed; 8 and 9 entry and exit on the 100 MHz counter; 10 tiles, 11 query row, 12 chunk index,
// 13 kernel (1 the 128-head kernel, 2 the head-split kernel). In the library proper the macros
// expand to nothing.
#ifdef MLA_PHASE_STAMPS
constexpr int kStampSlots = 16;
constexpr int kStampMaxWorkgroups = 8192;
__device__ unsigned long long g_phase_stamps[kStampMaxWorkgroups][kStampSlots];
__device__ __forceinline__ void phase_stamp(int slot, unsigned long long v) {
  const unsigned wg = blockIdx.x + blockIdx.y * gridDim.x;
  if (threadIdx.x == 0 && wg < (unsigned)kStampMaxWorkgroups) g_phase_stamps[wg][slot] = v;
}
#define MLA_STAMP(slot) phase_stamp(slot, __builtin_amdgcn_s_memtime())
#define MLA_STAMP_REAL(slot) phase_stamp(slot, __builtin_amdgcn_s_memrealtime())
#define MLA_STAMP_VAL(slot, v) phase_stamp(slot, (unsigned long long)(v))
#define MLA_STAMP_DRAIN() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")
#else
#define MLA_STAMP(slot) ((void)0)
#define MLA_STAMP_REAL(slot) ((void)0)
#define MLA_STAMP_VAL(slot, v) ((void)0)
#define MLA_STAMP_DRAIN() ((void)0)
#endif

// one 16-byte-per-lane direct global->LDS load: lane l writes LDS bytes lds_base + 16 l
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_vmcnt_9() { __builtin_amdgcn_s_waitcnt((9 & 15) | (7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_vmcnt_0() { __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8)); }
// vmcnt has six bits on gfx9: the low four at [3:0], the high two at [15:14]
__device__ __forceinline__ void wait_vmcnt_18() {
  __builtin_amdgcn_s_waitcnt((18 & 15) | ((18 >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt_27() {
  __builtin_amdgcn_s_waitcnt((27 & 15) | ((27 >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Split-K partials: per (query row, chunk) one block of H * DC accumulator values, stored as bf16
// (rounded once, to nearest even), and H (m, l) pairs in float32. The latent sums are accumulated in
// float32 in the registers; only their hand-over to the merge is rounded (at most 2^-9 relative per
// value, independent across chunks), which halves the partial traffic of every split row.
// The attention kernels store them in the accumulator's own register order, so they write them
// with whole 1 KB stores straight from the accumulators and attn_merge_frag reads them the same way:
//   [head block hb][col block cb (16)][row-group pair jp (2)][lane][8]
// holds O^T[col][head] for col = 32cb + 8j + 4(lane / 32) + e with j = 2jp + (i / 4), e = i % 4
// (i = 0..7 the position in the lane's 8 values), head = 32hb + lane % 32: a lane's 8 values are
// 8 consecutive accumulator registers.
// For mla_decode_step, decode_attn_hsplit stores them head-major instead, [head][col], so that one
// head's 1 KB row per chunk is contiguous for merge_heads_out_proj, which merges and projects one
// head per workgroup. The head-split kernel writes its (few, latency-bound) partials with
// nontemporal stores, which shortens the write-back at the end of the kernel; the big kernel's
// go through the caches (nontemporal stores measured slower on the ragged batch). attn_merge_frag
// reads every partial nontemporally: cached by the merge, the lines would slow the next call's
// stores.
constexpr int PART_ELEMS = H * DC;   // bf16 values per (query row, chunk)
__device__ __forceinline__ int frag_offset(int head, int col) {
  const int cb = col >> 5, j = (col >> 3) & 3, g = (col >> 2) & 1, e = col & 3;
  const int hb = head >> 5, lane = 32 * g + (head & 31);
  return ((((hb * 16 + cb) * 2 + (j >> 1)) * 64 + lane) * 8) + (j & 1) * 4 + e;
}
// eight float32 accumulator values rounded to bf16 (nearest even), packed for one 16-byte store
typedef float f32x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 lo, f32x4 hi) {
  const f32x8v v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, __builtin_convertvector(v, bf16x8v));
}
// the eight float32 values of a 16-byte bf16 piece
__device__ __forceinline__ void from_bf16x8(bf16x8 p, f32x4& lo, f32x4& hi) {
  const i32x4 u = __builtin_bit_cast(i32x4, p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = __uint_as_float((uint32_t)u[k] << 16), b = __uint_as_float((uint32_t)u[k] & 0xFFFF0000u);
    if (k < 2) { lo[2 * k] = a; lo[2 * k + 1] = b; } else { hi[2 * k - 4] = a; hi[2 * k - 3] = b; }
  }
}

// ---- How the keys are cut into chunks (one workgroup each).
// FIXED: the caller's n_splits, chunk k of row bt covers keys [k L, (k + 1) L) with
//   L = ceil(max_seq_len / n_splits); partial slot bt * n_splits + k.
// BALANCED (batch * n_q <= kBalanceRows): one grid of kBalanceGrid workgroups over the whole batch.
//   Q is the smallest bound (at least kMinTiles) for which cutting every row of t tiles into
//   ceil(t / Q) chunks needs at most kBalanceGrid chunks in all (found by bisection between
//   ceil(T / kBalanceGrid) and ceil(T / (kBalanceGrid - rows)), T the tiles of all rows), and each
//   row's tiles are split evenly over its chunks, so no chunk is longer than Q tiles whatever the
//   mix of lengths; the chunks of all rows are numbered in row order and chunk number =
//   workgroup = partial slot. (Ragged batch of 64 rows, 1K-8K keys: Q = 41 tiles where
//   ceil(T / (kBalanceGrid - rows)) gives 48.)
// PER_ROW: one chunk per row (many rows already fill the chip).
// HSPLIT (few rows and few keys, the latency-bound case): the BALANCED cut with kHsplitChunks
//   chunks of at least kHsplitMinTiles tiles, and four workgroups per chunk, one per head block of
//   32 heads (decode_attn_hsplit).
enum ChunkMode { FIXED = 0, BALANCED = 1, PER_ROW = 2, HSPLIT = 3 };
constexpr int kBalanceGrid = 256;
constexpr int kXcds = 8;   // MI355X: workgroup i runs on XCD i % 8
static_assert(kBalanceGrid % kXcds == 0, "the balanced grid splits evenly over the XCDs");
constexpr int kBalanceRows = 128;
constexpr int kMinTiles = 4;
constexpr int kHsplitChunks = 64;
constexpr int kHsplitMinTiles = 2;
constexpr int kHsplitRows = 16;
constexpr int kHsplitMaxTiles = 1024;   // rows x tiles of the longest row

struct Chunk {
  int bt, k, nck, slot, j0, j1;
};

// Inclusive prefix sum over the 64 lanes of a wave by DPP: row shifts by 1, 2, 4 and 8 scan each row
// of 16 lanes, then the broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3)
// carry the row totals across; no LDS round trip, unlike a shuffle. Lane 63 ends with the total.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// BALANCED plan over `grid` chunks of at least `min_tiles` tiles, computed by every lane of wave 0
// for all rows (rows <= 128: two per lane): the chunk numbered `target`. Returns false when
// `target` lies past the last chunk.
__device__ bool balanced_chunk(const int32_t* __restrict__ seq_len, int n_q, int rows, int target, int grid,
                               int min_tiles, Chunk* out) {
  const int lane = threadIdx.x & 63;
  int nvis[2], tiles[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = lane + 64 * u;
    const int b = n_q == 1 ? r : r / n_q, i = n_q == 1 ? 0 : r % n_q;   // one query row: no division
    nvis[u] = r < rows ? seq_len[b] - n_q + i + 1 : 0;
    tiles[u] = (nvis[u] + TILE - 1) / TILE;
  }
  // T, exactly: a lane's two rows hold under 2^27 tiles, so its count splits into 16-bit halves whose
  // sums over the wave fit 32 bits
  const int lsum = tiles[0] + tiles[1];
  const int64_t tsum = ((int64_t)__builtin_amdgcn_readlane(wave_scan_incl(lsum >> 16), 63) << 16) +
                       __builtin_amdgcn_readlane(wave_scan_incl(lsum & 0xFFFF), 63);
  // q: the smallest bound on a chunk's tiles for which every row cut into ceil(tiles / q) chunks
  // fits the grid. ceil(T / (grid - rows)) always fits (each row adds at most one partial
  // chunk), ceil(T / grid) is a lower bound, and the count only falls as q grows: bisect.
  const int64_t share = (tsum + (grid - rows) - 1) / (grid - rows);
  int lo = (int)max((int64_t)min_tiles, (tsum + grid - 1) / grid);
  int hi = (int)max((int64_t)min_tiles, share);
  while (lo < hi) {   // wave-uniform: lo, hi and the count (read from lane 63) are scalars
    const int mid = (lo + hi) / 2;
    // at most grid + rows chunks for any mid >= lo, so the sum cannot overflow
    const int cnt = __builtin_amdgcn_readlane(
        wave_scan_incl((tiles[0] + mid - 1) / mid + (tiles[1] + mid - 1) / mid), 63);
    if (cnt <= grid) hi = mid; else lo = mid + 1;
  }
  const int q = lo;
  bool found = false;
  int carry = 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int nck = (tiles[u] + q - 1) / q;
    const int incl = wave_scan_incl(nck);   // inclusive prefix over the 64 lanes of this round
    const int first = carry + incl - nck;
    const int r = lane + 64 * u;
    const bool mine = r < rows && target >= first && target < first + nck;
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;   // wave-uniform
      const int f = __builtin_amdgcn_readlane(first, src), n = __builtin_amdgcn_readlane(nck, src);
      const int nv = __builtin_amdgcn_readlane(nvis[u], src), nt = __builtin_amdgcn_readlane(tiles[u], src);
      const int k = target - f;
      // the row's tiles split evenly over its n chunks (sizes differ by at most one tile)
      const int t0 = (int)((int64_t)k * nt / n), t1 = (int)((int64_t)(k + 1) * nt / n);
      *out = Chunk{src + 64 * u, k, n, target, t0 * TILE, min(t1 * TILE, nv)};
      found = true;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return found;
}

// Exact fallback for one (query row, chunk) and heads h_begin .. h_end - 1: per head, a float32
// online softmax that rescales its running sum and latent accumulator at every block of 256 keys. Same outputs as the MFMA
// path (final z/lse with one chunk, otherwise a partial in log2 units). Kept out of line so the
// MFMA loop's register allocation does not see it.
__device__ __noinline__ void exact_chunk(const bf16* __restrict__ q_packed, const unsigned char* __restrict__ kv,
                                         size_t rh0, int j0, int j1, float scale_log2, int n_chunks, int slot,
                                         bf16* __restrict__ part_acc, float* __restrict__ part_ml,
                                         float* __restrict__ z, float* __restrict__ lse, unsigned char* smem,
                                         int h_begin, int h_end, bool head_major) {
  float* qs = reinterpret_cast<float*>(smem);   // [ROW]
  float* ps = qs + ROW;                         // [256]
  float* red = ps + 256;                        // [8]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int h = h_begin; h < h_end; ++h) {
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
      bf16* blk = part_acc + (size_t)slot * PART_ELEMS;
      blk[head_major ? h * DC + tid : frag_offset(h, tid)] = (bf16)acc0;
      blk[head_major ? h * DC + tid + 256 : frag_offset(h, tid + 256)] = (bf16)acc1;
      if (tid == 0) {
        part_ml[((size_t)slot * H + h) * 2 + 0] = m;
        part_ml[((size_t)slot * H + h) * 2 + 1] = l;
      }
    }
    __syncthreads();
  }
}

// grid: FIXED (n_splits, rows), BALANCED (kBalanceGrid), PER_ROW (rows); 256 threads,
// sizeof(Smem) dynamic LDS
__global__ void __launch_bounds__(256)
    decode_attn_fast(const bf16* __restrict__ q_packed, const bf16* __restrict__ cache,
                     const int64_t* __restrict__ seq_off, const int32_t* __restrict__ seq_len, int n_q, int rows,
                     float scale_log2, int mode, int n_splits, int chunk_len, bf16* __restrict__ part_acc,
                     float* __restrict__ part_ml, int2* __restrict__ row_chunks, float* __restrict__ z,
                     float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  MLA_STAMP(0);
  MLA_STAMP_REAL(8);
  MLA_STAMP_VAL(13, 1);

  // ---- this workgroup's chunk
  Chunk ch;
  if (mode == FIXED) {
    const int bt = blockIdx.y, k = blockIdx.x;
    const int n_vis = seq_len[bt / n_q] - n_q + (bt % n_q) + 1;
    ch = Chunk{bt, k, (n_vis + chunk_len - 1) / chunk_len, bt * n_splits + k, k * chunk_len,
               min((k + 1) * chunk_len, n_vis)};
    if (ch.j0 >= ch.j1) return;   // past the row's last chunk: nothing to do, nothing written
  } else if (mode == PER_ROW) {
    const int bt = blockIdx.x;
    ch = Chunk{bt, 0, 1, 0, 0, seq_len[bt / n_q] - n_q + (bt % n_q) + 1};
  } else {
    static_assert(FLAGS_OFF + 64 + sizeof(Chunk) <= LSUM_OFF, "the plan must end before the per-head sums");
    Chunk* shared_ch = reinterpret_cast<Chunk*>(smem_raw + FLAGS_OFF + 64);
    if (w == 0) {
      Chunk c;
      // Workgroups are dealt to the 8 XCDs in turn; numbering the chunks so that XCD x takes the 32
      // consecutive chunks 32x .. 32x + 31 puts the few workgroups of one row on one XCD, where they
      // share the row's 147 KB of queries through its L2 instead of each fetching them from HBM.
      const int target = (int)(blockIdx.x % kXcds) * (kBalanceGrid / kXcds) + (int)(blockIdx.x / kXcds);
      const bool found = balanced_chunk(seq_len, n_q, rows, target, kBalanceGrid, kMinTiles, &c);
      if (lane == 0) {
        if (!found) c.nck = 0;
        *shared_ch = c;
      }
    }
    __syncthreads();
    ch = *shared_ch;
    if (ch.nck == 0) return;   // the plan has fewer chunks than the grid
  }
  const int bt = ch.bt, j0 = ch.j0, j1 = ch.j1, n_chunks = ch.nck;
  const int b = bt / n_q;
  const size_t rh0 = (size_t)bt * H;
  MLA_STAMP(1);
  MLA_STAMP_VAL(10, (j1 - j0 + TILE - 1) / TILE);
  MLA_STAMP_VAL(11, bt);
  MLA_STAMP_VAL(12, ch.k);
  // every row's first chunk publishes where the row's partials are (first slot, count; count 1
  // means the row is written directly), so the merge never reads an entry of an earlier call
  if (row_chunks != nullptr && ch.k == 0 && threadIdx.x == 0) row_chunks[bt] = make_int2(ch.slot, n_chunks);
  const int n_tiles = (j1 - j0 + TILE - 1) / TILE;
  const unsigned char* kv = reinterpret_cast<const unsigned char*>(cache + seq_off[b] * (int64_t)ROW);
  // always-valid DMA source for "no tile left": this query row's packed queries (H * ROW_BYTES bytes)
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(q_packed + rh0 * ROW);

  // ---- DMA plan: slot (row r, physical chunk p) of the LDS tile is filled from logical chunk
  // phys_chunk(p, r) of key r: dma_off = r * ROW_BYTES + 16 * phys_chunk(p, r).
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int it = 0; it < DMA_PER_WAVE; ++it) {
    const int slot = w * SLOTS_PER_WAVE + it * 64 + lane;
    const int r = slot / ROW_CHUNKS, p = slot % ROW_CHUNKS;
    dma_off[it] = r * ROW_BYTES + phys_chunk(p, r) * 16 - (it % 4) * 1024 + DMA_BIAS;
  }
  auto tile_lds = [&](int tile) { return (uint32_t)(uintptr_t)MLA_LDS(unsigned char, sm.tile[tile % NBUF]); };
  // Where tile `tile` is read from (less DMA_BIAS), with the lane's offsets dma_off. A partial last
  // tile of a chunk of two or more tiles is moved back to end at the chunk's last key: its first
  // tail_shift rows repeat keys of the tile before, and their scores are masked. The move keeps
  // every read inside the chunk and the same for all lanes, so the loop passes dma_off to the DMA
  // untouched. (A chunk shorter than one tile cannot move back; its one tile re-reads its last key
  // instead, with per-lane offsets, in the prologue.) A tile past the chunk reads qbytes.
  const int tail_shift = n_tiles >= 2 ? j0 + n_tiles * TILE - j1 : 0;
  auto tile_src = [&](int tile) -> const unsigned char* {
    if (tile >= n_tiles) return qbytes - DMA_BIAS;
    const int key0 = j0 + tile * TILE - (tile == n_tiles - 1 ? tail_shift : 0);
    return kv + (int64_t)key0 * ROW_BYTES - DMA_BIAS;
  };
  auto sgpr_ptr = [](const void* p) {
    const uint64_t sb = (uint64_t)(uintptr_t)p;
    return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb);
  };
  // stand-alone tile DMA (prologue): nine 1 KB instructions per wave into the tile's buffer
  auto issue_tile = [&](int tile) {
    uint32_t o[DMA_PER_WAVE];
#pragma unroll
    for (int it = 0; it < DMA_PER_WAVE; ++it) o[it] = dma_off[it];
    if (n_tiles == 1 && tile == 0 && j1 - j0 < TILE) {   // lone partial tile: rows past the end re-read the last key
      const int last = j1 - 1 - j0;
#pragma unroll
      for (int it = 0; it < DMA_PER_WAVE; ++it) {
        const int r = (w * SLOTS_PER_WAVE + it * 64 + lane) / ROW_CHUNKS;
        o[it] = dma_off[it] - (r > last ? r - last : 0) * ROW_BYTES;
      }
    }
    const uint64_t sbase = sgpr_ptr(tile_src(tile));
    const uint32_t sdst = __builtin_amdgcn_readfirstlane(tile_lds(tile) + (w * SLOTS_PER_WAVE) * 16);
    asm volatile(
@DMA_ASM@
        ::[b] "s"(sbase), [m] "s"(sdst), [o0] "v"(o[0]), [o1] "v"(o[1]), [o2] "v"(o[2]), [o3] "v"(o[3]),
        [o4] "v"(o[4]), [o5] "v"(o[5]), [o6] "v"(o[6]), [o7] "v"(o[7]), [o8] "v"(o[8])
        : "memory", "m0");
  };

  // ---- queries of this wave's 32 heads (32w .. 32w+31).
  // Latent part: 32 B fragments (8 bf16 per lane: dims 16s + 8g .. +7 of head 32w + l32) for
  // v[128:255]. Loaded straight from global memory, every instruction would touch 32 rows 1152 B
  // apart, so the rows are staged through LDS instead: each wave copies its 32 rows with 1 KB
  // direct global->LDS loads (8 whole cache lines each) into slots QS_STRIDE bytes apart (the
  // 16-byte pad puts the 16 heads of one LDS phase on 16 different bank groups), then reads its
  // fragments. The staging area is the tile buffers, free until the first tile DMA.
  // Position part: 4 fragments per lane, loaded into v[64:79] for every score phase.
  const int qhead = w * 32 + l32;
  const bf16* qrow = q_packed + (rh0 + qhead) * ROW + 8 * g;
  const uint32_t qstage = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, &sm.tile[0][0]) + w * 32 * QS_STRIDE;
  {
    const unsigned char* qw = reinterpret_cast<const unsigned char*>(q_packed + (rh0 + w * 32) * ROW) + 16 * lane;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) dma16(qw + i * ROW_BYTES, __builtin_amdgcn_readfirstlane(qstage + i * QS_STRIDE));
  }
  i32x4 qrp0, qrp1, qrp2, qrp3;   // position part, dims 16s + 8g .. +7 of head qhead
  {
    const i32x4* qp = reinterpret_cast<const i32x4*>(qrow + DC);
    qrp0 = qp[0];
    qrp1 = qp[2];
    qrp2 = qp[4];
    qrp3 = qp[6];
  }
  wait_vmcnt_0();   // the staged rows are in
  v16i q0, q1, q2, q3, q4, q5, q6, q7;
  asm volatile(
@QLOAD_ASM@
      : "=&{v[128:143]}"(q0), "=&{v[144:159]}"(q1), "=&{v[160:175]}"(q2), "=&{v[176:191]}"(q3),
        "=&{v[192:207]}"(q4), "=&{v[208:223]}"(q5), "=&{v[224:239]}"(q6), "=&{v[240:255]}"(q7)
      : [a] "v"(qstage + l32 * QS_STRIDE + 16 * g)
      : "memory");
  lds_barrier();   // every wave holds its fragments: the staging area is free for the tiles
  MLA_STAMP(2);
  issue_tile(0);
  issue_tile(1);   // past the chunk when it has one tile: then a harmless read of qbytes
  MLA_STAMP(3);


  // O^T accumulators: latent col block cb (32 columns) x this wave's 32 heads, 16 fp32 each,
  // zeroed in AGPRs by MFMAs of zero operands (a plain zero initialisation would be built in
  // VGPRs first and copied over)
  f32x16 oc0, oc1, oc2, oc3, oc4, oc5, oc6, oc7, oc8, oc9, oc10, oc11, oc12, oc13, oc14, oc15;
  {
    // The zero operand is written by VALU just before: wait states before an MFMA reads it (the
    // compiler does not pad hazards into inline asm).
    const bf16x8 zf = {};
    asm volatile(
        "s_nop 7\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %1, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %3, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %4, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %5, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %6, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %7, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %8, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %9, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %10, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %11, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %12, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %13, %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %14, %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %15, %[z], %[z], 0"
        : "=a"(oc0), "=a"(oc1), "=a"(oc2), "=a"(oc3), "=a"(oc4), "=a"(oc5), "=a"(oc6), "=a"(oc7),
          "=a"(oc8), "=a"(oc9), "=a"(oc10), "=a"(oc11), "=a"(oc12), "=a"(oc13), "=a"(oc14), "=a"(oc15)
        : [z] "v"(zf));
  }

  float m_ref = -INFINITY;  // per lane: head 32w + l32 (both lane halves agree); set by the first tile
  float neg_mref = INFINITY;
  float l_run = 0.0f;       // per lane: sum over this lane's half of the keys
  // P buffers: lane l reads B fragment (head block hb, key step s) at pb + (2 hb + s) KB and writes
  // its own head block's two fragments at pw (+ 1 KB for the second key step)
  const uint32_t pbuf_lds = (uint32_t)(uintptr_t)MLA_LDS(unsigned char, &sm.pbuf[0][0]) + 16 * lane;
  auto p_read = [&](int tile) { return pbuf_lds + (tile & 1) * PBUF_BYTES; };
  auto p_write = [&](int tile) { return pbuf_lds + (tile & 1) * PBUF_BYTES + w * 2048; };

  // per-lane LDS byte offsets
  // scores: A operand row l32 = key pi(l32), logical chunk 2s + g -> phys (s/4)*8 + ((2(s%4)+g) ^ swz(key))
  uint32_t qk_off[4];
  {
    const int key = key_of_row(l32);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qk_off[s4] = key * ROW_BYTES + (((2 * s4 + g) ^ swz(key)) & 7) * 16;
  }
  // values: transpose reads of this wave's column blocks cb = 4w + db. lane = 16q + L;
  // row = 16s + 8g + 4h + L/4; col = 32cb + 16(q&1) + 4(L&3). Chunk group cb/2 = 2w + db/2: the
  // wave's 256 bytes are in the offsets, db/2 in the instruction's offset field.
  const int q16 = lane >> 4, L = lane & 15;
  uint32_t pv_off[2][2];  // [db & 1][h]
#pragma unroll
  for (int cbo = 0; cbo < 2; ++cbo)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g + 4 * h + (L >> 2);
      const int clow = 4 * cbo + 2 * (q16 & 1) + ((L >> 1) & 1);  // logical chunk & 7
      const int ph = (clow ^ swz(row)) & 7;
      pv_off[cbo][h] = row * ROW_BYTES + w * 256 + ph * 16 + (L & 1) * 8;
    }

  // Scores of one tile into v[112:127]. The same asm block issues the DMA of the tile two
  // after it (9 global_load_lds spread between the MFMAs, so the VMEM issue overlaps the matrix
  // work). That tile's buffer held the tile before the one being accumulated, which every wave
  // finished reading before the barrier that opened this iteration.
  auto scores = [&](int tile, f32x16& sacc) {
    const uint32_t tb = tile_lds(tile);
    const int dt = tile + 2;   // at least 2: never the lone partial tile
    const uint64_t sbase = sgpr_ptr(tile_src(dt));
    const uint32_t sdst = __builtin_amdgcn_readfirstlane(tile_lds(dt) + (w * SLOTS_PER_WAVE) * 16);
    asm volatile(
@QK_ASM@
        : "=&{v[112:127]}"(sacc)
        : [k0] "v"(tb + qk_off[0]), [k1] "v"(tb + qk_off[1]), [k2] "v"(tb + qk_off[2]), [k3] "v"(tb + qk_off[3]),
          "{v[64:67]}"(qrp0), "{v[68:71]}"(qrp1), "{v[72:75]}"(qrp2), "{v[76:79]}"(qrp3),
          "{v[128:143]}"(q0), "{v[144:159]}"(q1), "{v[160:175]}"(q2), "{v[176:191]}"(q3),
          "{v[192:207]}"(q4), "{v[208:223]}"(q5), "{v[224:239]}"(q6), "{v[240:255]}"(q7),
          [b] "s"(sbase), [m] "s"(sdst), [o0] "v"(dma_off[0]), [o1] "v"(dma_off[1]), [o2] "v"(dma_off[2]),
          [o3] "v"(dma_off[3]), [o4] "v"(dma_off[4]), [o5] "v"(dma_off[5]), [o6] "v"(dma_off[6]),
          [o7] "v"(dma_off[7]), [o8] "v"(dma_off[8])
        : "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87", "v88", "v89", "v90", "v91", "v92", "v93", "v94",
          "v95", "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108",
          "v109", "v110", "v111", "memory", "m0");
  };

  // softmax of the chunk's first tile in C++: fixes the reference, masks the rows past the end of a
  // chunk shorter than one tile (the only first tile that can be partial), and stores P (the
  // lane's two B fragments) to this wave's part of P buffer 0.
  auto softmax_first = [&](f32x16 sacc) {
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sv = (j0 + key_of_reg(r, g) < j1) ? sacc[r] * scale_log2 : -INFINITY;
      sacc[r] = sv;
      tmax = fmaxf(tmax, sv);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    m_ref = tmax;
    float psum = 0.0f;
    i32x4 pf[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2f(sacc[r] - m_ref), p1 = exp2f(sacc[r + 1] - m_ref);
      psum += p0 + p1;
      pf[r / 8][(r / 2) % 4] = (int)((uint32_t)__builtin_bit_cast(unsigned short, (bf16)p0) |
                                     ((uint32_t)__builtin_bit_cast(unsigned short, (bf16)p1) << 16));
    }
    unsigned char* pw = &sm.pbuf[0][0] + w * 2048 + 16 * lane;   // p_write(0)
    *reinterpret_cast<i32x4*>(pw) = pf[0];
    *reinterpret_cast<i32x4*>(pw + 1024) = pf[1];
    l_run += psum;
    neg_mref = -m_ref;
    asm volatile("" : "+v"(neg_mref));   // kept, not recomputed from m_ref in every tile
  };

  // P.V of tile t (P of all heads in P buffer t & 1) with the softmax of tile t+1 (scores in
  // v[112:127]) interleaved; stores P of tile t+1 to this wave's part of P buffer (t + 1) & 1, which
  // every wave finished reading (tile t-1) before the barrier that opened this iteration.
  auto pv_softmax = [&](int tile, f32x16& sacc) {
    const uint32_t tb = tile_lds(tile);
    asm volatile(
@PVSM_ASM@
        : [o0] "+a"(oc0), [o1] "+a"(oc1), [o2] "+a"(oc2), [o3] "+a"(oc3), [o4] "+a"(oc4), [o5] "+a"(oc5),
          [o6] "+a"(oc6), [o7] "+a"(oc7), [o8] "+a"(oc8), [o9] "+a"(oc9), [o10] "+a"(oc10), [o11] "+a"(oc11),
          [o12] "+a"(oc12), [o13] "+a"(oc13), [o14] "+a"(oc14), [o15] "+a"(oc15), [l] "+v"(l_run),
          "+{v[112:127]}"(sacc)
        : [v00] "v"(tb + pv_off[0][0]), [v01] "v"(tb + pv_off[0][1]), [v10] "v"(tb + pv_off[1][0]),
          [v11] "v"(tb + pv_off[1][1]), [sc] "s"(scale_log2), [nm] "v"(neg_mref), [pb] "v"(p_read(tile)),
          [pw] "v"(p_write(tile + 1))
        : "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87", "v88", "v89", "v90", "v91", "v92", "v93", "v94",
          "v95", "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104", "v105", "v106", "v107", "v108",
          "v109", "v110", "v111", "memory");
  };

  // ---- the loop. Iteration t >= 0: P.V of tile t fused with the softmax of tile t+1 (its scores
  // computed just before); iteration -1 only scores tile 0 and fixes the reference in C++.
  // Exactly one site per asm phase keeps the register assignment simple for the compiler.
  // Every score phase issues exactly one tile DMA (a harmless one past the chunk), so at the top
  // of each iteration the newest nine loads of this wave belong to the tile after next.
  for (int tile = -1; tile < n_tiles; ++tile) {
    wait_vmcnt_9();   // tile t+1 landed; tile t+2 may still be in flight
    lds_barrier();    // tile t+1 visible to all waves; iteration t-1 finished everywhere
    f32x16 sacc;
    if (tile + 1 < n_tiles) scores(tile + 1, sacc);
    if (tile < 0) {
      softmax_first(sacc);
      continue;
    }
    if (tile + 1 >= n_tiles) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = -INFINITY;   // no next tile: the fused softmax adds 0
    } else if (tile + 2 == n_tiles && tail_shift > 0) {   // the moved-back last tile: mask its repeated keys
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key_of_reg(r, g) < tail_shift) sacc[r] = -INFINITY;
    }
    pv_softmax(tile, sacc);
  }
  wait_vmcnt_0();   // the trailing DMAs (past the chunk) have landed; LDS is free
  MLA_STAMP(4);

  // A score far above the reference makes later probabilities overflow (inf / NaN in the
  // accumulator, harmless to the hardware); the loop still runs to its end, and the chunk is then
  // recomputed by the exact path. Every probability is at most the lane's sum l_run, so a sum of at
  // most 2^HEADROOM proves that no score exceeded the reference by more than HEADROOM; a larger (or
  // non-finite) sum sends the chunk to the exact path, which is correct for any input. The flags
  // meet in LDS once, after the loop.
  const bool ovf = __any(!(l_run <= kSumLimit));
  int* flags = reinterpret_cast<int*>(smem_raw + FLAGS_OFF);
  if (lane == 0) flags[w] = ovf ? 1 : 0;
  __syncthreads();
  const bool overflowed = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  if (overflowed) {
    __syncthreads();
    exact_chunk(q_packed, kv, rh0, j0, j1, scale_log2, n_chunks, ch.slot, part_acc, part_ml, z, lse, smem_raw, 0, H,
                false);
    return;
  }
  // the accumulator is read by VALU below: 20 wait states after the last MFMA
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(oc0), "+a"(oc1), "+a"(oc2), "+a"(oc3), "+a"(oc4), "+a"(oc5), "+a"(oc6), "+a"(oc7),
                 "+a"(oc8), "+a"(oc9), "+a"(oc10), "+a"(oc11), "+a"(oc12), "+a"(oc13), "+a"(oc14), "+a"(oc15));

  // ---- per-head totals: combine the two key halves of this lane's head
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    if (n_chunks == 1) {
      if (lse != nullptr) lse[rh0 + qhead] = (m_ref + log2f(l_run)) * kLn2;
    } else {
      float* ml = part_ml + ((size_t)ch.slot * H + qhead) * 2;
      ml[0] = m_ref;
      ml[1] = l_run;
    }
  }
  // accumulator db * 4 + hb: latent columns 32 (4w + db) .. +31 x heads 32 hb .. 32 hb + 31
  const f32x16* oacc[16] = {&oc0, &oc1, &oc2, &oc3, &oc4, &oc5, &oc6, &oc7,
                            &oc8, &oc9, &oc10, &oc11, &oc12, &oc13, &oc14, &oc15};
  if (n_chunks > 1) {
    // ---- partial: 32 stores of 1 KB per wave, straight from the accumulators (layout above:
    // head block hb, column block cb, half jp, lane)
    bf16* blk = part_acc + (size_t)ch.slot * PART_ELEMS + 8 * lane;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const f32x16& o = *oacc[db * 4 + hb];
          *reinterpret_cast<bf16x8*>(blk + (size_t)hb * (PART_ELEMS / 4) + ((4 * w + db) * 2 + jp) * 512) =
              to_bf16x8(f32x4{o[8 * jp], o[8 * jp + 1], o[8 * jp + 2], o[8 * jp + 3]},
                        f32x4{o[8 * jp + 4], o[8 * jp + 5], o[8 * jp + 6], o[8 * jp + 7]});
        }
    MLA_STAMP_DRAIN();
    MLA_STAMP(5);
    MLA_STAMP_REAL(9);
    return;
  }

  // ---- z = O / l: this wave holds latent columns 128w .. 128w+127 of every head. Each head's sum
  // l comes from the wave that scored it, through LDS. One head block at a time goes through this
  // wave's own slice of LDS: written straight from the accumulator layout, every store would touch
  // 32 rows; transposed, each store writes the wave's 512 bytes of two heads' rows.
  float* lsh = reinterpret_cast<float*>(smem_raw + LSUM_OFF);   // [H]
  if (g == 0) lsh[qhead] = l_run;
  __syncthreads();
  float inv[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) inv[hb] = 1.0f / lsh[32 * hb + l32];
  float* stage = reinterpret_cast<float*>(smem_raw) + w * 32 * ES_STRIDE;   // [32 heads][ES_STRIDE]
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    float* row = stage + l32 * ES_STRIDE + 4 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& o = *oacc[db * 4 + hb];
        *reinterpret_cast<f32x4*>(row + 32 * db + 8 * j) =
            f32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]} * inv[hb];
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's writes land before its reads
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int hr = 2 * i + g;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + hr * ES_STRIDE + 4 * l32);
      *reinterpret_cast<f32x4*>(z + (rh0 + 32 * hb + hr) * DC + 128 * w + 4 * l32) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next block's writes
  }
  MLA_STAMP_DRAIN();
  MLA_STAMP(5);
  MLA_STAMP_REAL(9);
}

// ---- Head-split kernel for few query rows and short histories (latency-bound decode).
// Four workgroups share each chunk, one per head block hb of 32 heads; inside a workgroup the
// 4 waves split both contractions instead of the heads: wave w scores the 32 keys of a tile
// against its 32 heads over dims 144w .. 144w+143 (9 MFMA k-steps), the four partial score tiles
// meet in LDS, every wave runs the same softmax on their sum (added in wave order, so all waves
// hold bitwise the same probabilities), and wave w accumulates latent columns 128w .. 128w+127
// (col blocks 4w .. 4w+3). Per tile a wave issues 17 MFMAs instead of 68, so a chunk of a few
// tiles finishes in a fraction of the big kernel's time, the queries a workgroup stages are 36 KB
// instead of 147 KB, and the split-K partials come out 4x fewer for the same number of
// workgroups. The price is that each cache tile is streamed into four workgroups; they run on
// the same XCD, so three of the four reads hit its L2. Same tile layout (swizzled DMA),
// fixed-reference softmax with the exact fallback and partial layout as decode_attn_fast, or, with
// head_major, the head-major partials that merge_heads_out_proj reads.
typedef __bf16 bf16x8e __attribute__((ext_vector_type(8)));
typedef short i16x4e __attribute__((ext_vector_type(4)));
typedef float f32x16e __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
typedef float f32x2e __attribute__((ext_vector_type(2)));

// LDS (all 160 KB): tile t being computed on, t+1 .. t+3 in flight (the queries are staged in the
// buffer of tile 3), and the partial-score exchange
constexpr int HS_NBUF = 4;
struct SmemH {
  unsigned char tile[HS_NBUF][TILE_BYTES];
  float exch[WAVES][4][64][4];   // partial scores: [wave][register quad][lane][4]
};
static_assert(sizeof(SmemH) <= 160 * 1024, "LDS budget");
constexpr int HS_STAGE = DC + 4;   // floats per staged partial row (the pad spreads 16 heads over the banks)
static_assert(32 * HS_STAGE * 4 <= HS_NBUF * TILE_BYTES, "partial staging fits the tile buffers");

__device__ __forceinline__ f32x16e mfma_bf16(bf16x8e a, bf16x8e b, f32x16e c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte operand piece of logical chunk c (8 dims) of tile row r
__device__ __forceinline__ bf16x8e row_piece(const unsigned char* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8e*>(tile + r * ROW_BYTES + phys_chunk(c, r) * 16);
}

// A operand V^T (32 latent columns of block cb x 16 keys of step s) by two transpose reads: lane
// l = 16q + L gets tile[16s + 8g + e][32cb + l % 32], e = 0..7; source lane L of its 16-lane group
// points at row 16s + 8g + 4h + L/4, columns 32cb + 16(q & 1) + 4(L & 3) .. +3, halves h = 0, 1.
__device__ __forceinline__ bf16x8e v_fragment(const unsigned char* tile, int s, int cb, int lane) {
  const int g = lane >> 5, q = lane >> 4, L = lane & 15;
  const int c = 4 * cb + 2 * (q & 1) + ((L >> 1) & 1);   // logical 16-byte chunk of the 4 columns
  i16x4e hv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * s + 8 * g + 4 * h + (L >> 2);
    const unsigned char* p = tile + r * ROW_BYTES + phys_chunk(c, r) * 16 + 8 * (L & 1);
    hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4e*)MLA_LDS(unsigned char, p));
  }
  return __builtin_bit_cast(bf16x8e, hv);
}

// The BALANCED cut for the head-split grid (kHsplitChunks chunks of at least kHsplitMinTiles
// tiles), computed by every lane from uniform loads of seq_len (scalar loads, so they wait on
// lgkmcnt and never on the tile DMAs in flight): the chunk numbered `target`, or false when the
// plan has fewer chunks. rows <= kHsplitRows.
__device__ __forceinline__ bool hsplit_chunk(const int32_t* __restrict__ seq_len, int n_q, int rows, int target,
                                             Chunk* out) {
  int total = 0;
  for (int r = 0; r < rows; ++r) total += (seq_len[r / n_q] - n_q + (r % n_q) + 1 + TILE - 1) / TILE;
  const int q = max(kHsplitMinTiles, (total + (kHsplitChunks - rows) - 1) / (kHsplitChunks - rows));
  int first = 0;
  for (int r = 0; r < rows; ++r) {
    const int nvis = seq_len[r / n_q] - n_q + (r % n_q) + 1;
    const int nck = ((nvis + TILE - 1) / TILE + q - 1) / q;
    if (target < first + nck) {
      const int k = target - first;
      *out = Chunk{r, k, nck, target, k * q * TILE, min((k + 1) * q * TILE, nvis)};
      return true;
    }
    first += nck;
  }
  return false;
}

// grid: 4 * kHsplitChunks workgroups, 256 threads, sizeof(SmemH) dynamic LDS
__global__ void __launch_bounds__(256)
    decode_attn_hsplit(const bf16* __restrict__ q_packed, const bf16* __restrict__ cache,
                       const int64_t* __restrict__ seq_off, const int32_t* __restrict__ seq_len, int n_q, int rows,
                       float scale_log2, bf16* __restrict__ part_acc, float* __restrict__ part_ml,
                       int2* __restrict__ row_chunks, float* __restrict__ z, float* __restrict__ lse,
                       int head_major) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SmemH& sm = *reinterpret_cast<SmemH*>(smem_raw);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // Workgroups are dealt to the 8 XCDs in turn: the four head blocks of chunk 8a + x are
  // workgroups 32a + 8hb + x, all on XCD x.
  const int wg = blockIdx.x;
  const int hb = (wg >> 3) & 3, cidx = ((wg >> 5) << 3) | (wg & 7);
  const int head0 = 32 * hb;
  MLA_STAMP(0);
  MLA_STAMP_REAL(8);
  MLA_STAMP_VAL(13, 2);

  // DMA plan as in decode_attn_fast: slot (row r, physical chunk p) <- logical chunk phys_chunk(p, r)
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int it = 0; it < DMA_PER_WAVE; ++it) {
    const int slot = w * SLOTS_PER_WAVE + it * 64 + lane;
    const int r = slot / ROW_CHUNKS, p = slot % ROW_CHUNKS;
    dma_off[it] = r * ROW_BYTES + phys_chunk(p, r) * 16;
  }
  auto buf_lds = [&](int buf) { return (uint32_t)(uintptr_t)MLA_LDS(unsigned char, sm.tile[buf]); };
  // 32 rows of 1152 bytes from `src` (rows past `last` re-read row `last`) into buffer `buf`
  auto dma_rows = [&](const unsigned char* src, int last, int buf) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(buf_lds(buf) + (w * SLOTS_PER_WAVE) * 16);
#pragma unroll
    for (int it = 0; it < DMA_PER_WAVE; ++it) {
      const int r = dma_off[it] / ROW_BYTES;
      const uint32_t o = dma_off[it] - (r > last ? r - last : 0) * ROW_BYTES;
      dma16(src + o, dst + it * 1024);
    }
  };
  // queries of heads head0 .. head0+31 (32 contiguous rows), staged like a tile in buffer 3. With
  // one query row the row is known before the plan, and the load overlaps it.
  auto stage_queries = [&](int bt) {
    dma_rows(reinterpret_cast<const unsigned char*>(q_packed + ((size_t)bt * H + head0) * ROW), TILE - 1, 3);
  };
  if (rows == 1) stage_queries(0);
  // sequence 0's slab offset is loaded next to the plan's lengths rather than after it: with one
  // sequence (the latency-bound case) the tile addresses then wait for one memory round trip
  const int64_t off0 = seq_off[0];
  Chunk ch;
  if (!hsplit_chunk(seq_len, n_q, rows, cidx, &ch)) {   // the plan has fewer chunks than the grid
    wait_vmcnt_0();   // no LDS load may land after the workgroup has ended
    return;
  }
  const int bt = ch.bt, j0 = ch.j0, j1 = ch.j1, n_chunks = ch.nck;
  const int b = bt / n_q;
  const size_t rh0 = (size_t)bt * H;
  MLA_STAMP(1);
  MLA_STAMP_VAL(10, (j1 - j0 + TILE - 1) / TILE);
  MLA_STAMP_VAL(11, bt);
  MLA_STAMP_VAL(12, ch.k);
  if (row_chunks != nullptr && ch.k == 0 && hb == 0 && threadIdx.x == 0) row_chunks[bt] = make_int2(ch.slot, n_chunks);
  const int n_tiles = (j1 - j0 + TILE - 1) / TILE;
  const unsigned char* kv = reinterpret_cast<const unsigned char*>(cache + (b == 0 ? off0 : seq_off[b]) * (int64_t)ROW);
  auto issue_tile = [&](int tile) {
    const int key0 = j0 + tile * TILE;
    dma_rows(kv + (int64_t)key0 * ROW_BYTES, min(TILE, j1 - key0) - 1, tile % HS_NBUF);
  };

  // queries (unless already in flight), then up to three tiles; vmcnt counts in issue order, so
  // once at most 9 x (tiles issued) loads are outstanding the queries have landed
  if (rows != 1) stage_queries(bt);
  issue_tile(0);
  if (n_tiles > 2) {
    issue_tile(1);
    issue_tile(2);
    wait_vmcnt_27();
  } else if (n_tiles > 1) {
    issue_tile(1);
    wait_vmcnt_18();
  } else {
    wait_vmcnt_9();
  }
  lds_barrier();
  MLA_STAMP(3);
  // B operand of the scores: head l32, dims 16s + 8g .. +7 for this wave's k-steps s = 9w + u
  bf16x8e qf[9];
#pragma unroll
  for (int u = 0; u < 9; ++u) qf[u] = row_piece(sm.tile[3], l32, 2 * (9 * w + u) + g);
  const int akey = key_of_row(l32);   // A operand row l32 holds key pi(l32)

  f32x16e oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16e{};
  float m_ref = -INFINITY, l_run = 0.0f;
  bool ovf = false;
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 2 < n_tiles)   // tile t landed; tiles t+1 and t+2 may still be in flight
      wait_vmcnt_18();
    else if (t + 1 < n_tiles)
      wait_vmcnt_9();
    else
      wait_vmcnt_0();
    lds_barrier();      // tile t visible; iteration t-1 (and the query reads) finished everywhere
    if (t + 3 < n_tiles) issue_tile(t + 3);   // into the buffer of tile t-1 (or of the queries)
    const unsigned char* tb = sm.tile[t % HS_NBUF];
    f32x16e sp = f32x16e{};
#pragma unroll
    for (int u = 0; u < 9; ++u) sp = mfma_bf16(row_piece(tb, akey, 2 * (9 * w + u) + g), qf[u], sp);
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      *reinterpret_cast<f32x4*>(&sm.exch[w][qd][lane][0]) = f32x4{sp[4 * qd], sp[4 * qd + 1], sp[4 * qd + 2], sp[4 * qd + 3]};
    lds_barrier();
    float sv[16];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      f32x4 v = *reinterpret_cast<const f32x4*>(&sm.exch[0][qd][lane][0]);
#pragma unroll
      for (int u = 1; u < WAVES; ++u) v += *reinterpret_cast<const f32x4*>(&sm.exch[u][qd][lane][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[4 * qd + e] = v[e] * scale_log2;
    }
    // softmax against the chunk's fixed reference (the first tile's maximum), keys past the end
    // of a tail tile masked
    const int key0 = j0 + t * TILE;
    if (key0 + TILE > j1) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + key_of_reg(r, g) >= j1) sv[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    if (t == 0) {
      m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
    } else {
      ovf |= mx > m_ref + HEADROOM;
    }
    int pk[8];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {   // 2^x of the hardware (results below 2^-126 flush to 0)
      const float p0 = __builtin_amdgcn_exp2f(sv[r] - m_ref), p1 = __builtin_amdgcn_exp2f(sv[r + 1] - m_ref);
      psum += p0 + p1;
      pk[r / 2] = __builtin_bit_cast(int, __builtin_convertvector((f32x2e){p0, p1}, bf16x2e));
    }
    l_run += psum;
    // P^T B fragments: keys 16s + 8g + e of this lane's head are score registers 8s + e
    const int pk0[4] = {pk[0], pk[1], pk[2], pk[3]}, pk1[4] = {pk[4], pk[5], pk[6], pk[7]};
    const bf16x8e pb0 = __builtin_bit_cast(bf16x8e, pk0), pb1 = __builtin_bit_cast(bf16x8e, pk1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cb = 4 * w + i;
      oacc[i] = mfma_bf16(v_fragment(tb, 0, cb, lane), pb0, oacc[i]);
      oacc[i] = mfma_bf16(v_fragment(tb, 1, cb, lane), pb1, oacc[i]);
    }
  }

  // every wave ran the same softmax, so the flags agree; they still meet in LDS once
  int* flags = reinterpret_cast<int*>(&sm.exch[0][0][0][0]);
  const bool wave_ovf = __any(ovf);
  lds_barrier();   // every wave is done with the exchange area
  MLA_STAMP(4);
  if (lane == 0) flags[w] = wave_ovf ? 1 : 0;
  __syncthreads();
  if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) {
    __syncthreads();
    exact_chunk(q_packed, kv, rh0, j0, j1, scale_log2, n_chunks, ch.slot, part_acc, part_ml, z, lse, smem_raw, head0,
                head0 + 32, head_major != 0);
    return;
  }
  l_run += __shfl_xor(l_run, 32, 64);
  const int head = head0 + l32;
  if (n_chunks == 1) {
    // z = O / l: lane (g, head) holds columns 32cb + 8j + 4g .. +3
    const float inv = 1.0f / l_run;
    float* zr = z + (rh0 + head) * DC + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(zr + 32 * (4 * w + i) + 8 * j) =
            f32x4{oacc[i][4 * j], oacc[i][4 * j + 1], oacc[i][4 * j + 2], oacc[i][4 * j + 3]} * inv;
    if (lse != nullptr && w == 0 && g == 0) lse[rh0 + head] = (m_ref + log2f(l_run)) * kLn2;
    MLA_STAMP_DRAIN();
    MLA_STAMP(5);
    MLA_STAMP_REAL(9);
    return;
  }
  if (head_major) {
    // head-major partial, staged through the (now idle) tile buffers: each lane holds 32-byte
    // pieces of 16 head rows, so the rows are assembled in LDS first and then leave as whole 1 KB
    // stores
    float* stage = reinterpret_cast<float*>(&sm.tile[0][0]);   // [32 heads][HS_STAGE]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(stage + l32 * HS_STAGE + 32 * (4 * w + i) + 8 * j + 4 * g) =
            f32x4{oacc[i][4 * j], oacc[i][4 * j + 1], oacc[i][4 * j + 2], oacc[i][4 * j + 3]};
    __syncthreads();
    // each lane rounds 8 consecutive columns of a head row: one 1 KB store per row
    bf16* prow = part_acc + (size_t)ch.slot * PART_ELEMS + (size_t)head0 * DC + 8 * lane;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int hl = 8 * w + hh;
      const float* sr = stage + hl * HS_STAGE + 8 * lane;
      const bf16x8 v = to_bf16x8(*reinterpret_cast<const f32x4*>(sr), *reinterpret_cast<const f32x4*>(sr + 4));
      __builtin_nontemporal_store(__builtin_bit_cast(i32x4, v), reinterpret_cast<i32x4*>(prow + (size_t)hl * DC));
    }
  } else {
    // register-order partial: 1 KB stores straight from the accumulators
    bf16* blk = part_acc + (size_t)ch.slot * PART_ELEMS + (size_t)hb * (PART_ELEMS / 4) + 8 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const bf16x8 v = to_bf16x8(f32x4{oacc[i][8 * jp], oacc[i][8 * jp + 1], oacc[i][8 * jp + 2], oacc[i][8 * jp + 3]},
                                   f32x4{oacc[i][8 * jp + 4], oacc[i][8 * jp + 5], oacc[i][8 * jp + 6], oacc[i][8 * jp + 7]});
        __builtin_nontemporal_store(__builtin_bit_cast(i32x4, v),
                                    reinterpret_cast<i32x4*>(blk + ((4 * w + i) * 2 + jp) * 512));
      }
  }
  if (w == 0 && g == 0) {
    float* ml = part_ml + ((size_t)ch.slot * H + head) * 2;
    ml[0] = m_ref;
    ml[1] = l_run;
  }
  MLA_STAMP_DRAIN();
  MLA_STAMP(5);
  MLA_STAMP_REAL(9);
}

// Log-sum-exp merge of decode_attn_fast's split-K partials (register order, bf16). One workgroup per
// (query row, head block hb, col block cb, JP of the 2 row-group pairs jp): 32 heads x 16 JP latent
// columns, each lane owning one head and 8 JP columns (JP = 2 for many rows; JP = 1 spreads a few
// rows over twice as many workgroups). The row's chunks are the slots base .. base + nck - 1 (every
// one saw at least one key), as published by the row's first chunk.
// With M = max_k m_k (m in log2 units), z = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k.
// One pass: the 4 waves take the chunks round-robin, CU chunks (coalesced 1 KB loads of the
// partial and its (m, l)) in flight per step, and each wave keeps its own running maximum,
// rescaling its sums when it grows; the wave sums then meet in LDS against the common maximum.
// Rows computed as a single chunk were written directly and are skipped.
template <int JP>
__global__ void __launch_bounds__(256) attn_merge_frag(const bf16* __restrict__ part_acc,
                                                       const float* __restrict__ part_ml,
                                                       const int2* __restrict__ row_chunks,
                                                       float* __restrict__ z, float* __restrict__ lse) {
  constexpr int CU = JP == 1 ? 16 : 4;   // chunks per step and wave
  __shared__ f32x4 red[3][JP][2][64];
  __shared__ float lred[3][64];
  __shared__ float mred[3][64];
  const int bt = blockIdx.y;
  const int slab = blockIdx.x / (2 / JP), jpbase = (blockIdx.x % (2 / JP)) * JP;   // slab = hb * 16 + cb
  const int hb = slab >> 4, cb = slab & 15;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, hl = lane & 31;
  const int2 rc = row_chunks[bt];
  if (rc.y <= 1) return;
  const int base = rc.x, nck = rc.y;
  const size_t head = (size_t)32 * hb + hl;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + (size_t)base * H + head;   // stride H
  const bf16* src = part_acc + (size_t)base * PART_ELEMS + (size_t)slab * 1024 + (size_t)jpbase * 512 + 8 * lane;
  float m_w = -INFINITY, Lsum = 0.0f;
  f32x4 acc[JP][2] = {};
  for (int k0 = wv; k0 < nck; k0 += 4 * CU) {   // chunk k0 exists, so every step sees one
    i32x4 x[CU][JP];
    float2 v[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int kk = k0 + 4 * u;
      v[u] = make_float2(-INFINITY, 0.0f);
      if (kk < nck) {
#pragma unroll
        for (int j = 0; j < JP; ++j) {
          const i32x4* p = reinterpret_cast<const i32x4*>(src + (size_t)kk * PART_ELEMS + j * 512);
          x[u][j] = __builtin_nontemporal_load(p);
        }
        v[u] = ml[(size_t)kk * H];
      }
    }
    float mb = m_w;
#pragma unroll
    for (int u = 0; u < CU; ++u) mb = fmaxf(mb, v[u].x);
    const float a = exp2f(m_w - mb);   // 0 on the first step (m_w = -inf, mb finite)
    Lsum *= a;
#pragma unroll
    for (int j = 0; j < JP; ++j) {
      acc[j][0] *= a;
      acc[j][1] *= a;
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      if (k0 + 4 * u < nck) {
        const float wk = exp2f(v[u].x - mb);
        Lsum = fmaf(wk, v[u].y, Lsum);
#pragma unroll
        for (int j = 0; j < JP; ++j) {
          f32x4 lo, hi;
          from_bf16x8(__builtin_bit_cast(bf16x8, x[u][j]), lo, hi);
          acc[j][0] += wk * lo;
          acc[j][1] += wk * hi;
        }
      }
    }
    m_w = mb;
  }
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < JP; ++j) {
      red[wv - 1][j][0][lane] = acc[j][0];
      red[wv - 1][j][1][lane] = acc[j][1];
    }
    lred[wv - 1][lane] = Lsum;
    mred[wv - 1][lane] = m_w;
  }
  __syncthreads();
  if (wv == 0) {
    // wave 0 always holds chunk 0, so M is finite; a wave without chunks weighs 2^-inf = 0
    float M = m_w;
#pragma unroll
    for (int u = 0; u < 3; ++u) M = fmaxf(M, mred[u][lane]);
    const float a0 = exp2f(m_w - M);
    Lsum *= a0;
#pragma unroll
    for (int j = 0; j < JP; ++j) {
      acc[j][0] *= a0;
      acc[j][1] *= a0;
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const float au = exp2f(mred[u][lane] - M);
      Lsum = fmaf(au, lred[u][lane], Lsum);
#pragma unroll
      for (int j = 0; j < JP; ++j) {
        acc[j][0] += au * red[u][j][0][lane];
        acc[j][1] += au * red[u][j][1][lane];
      }
    }
    // the two lane halves of a head summed the same chunks: Lsum agrees between them
    const size_t rh = (size_t)bt * H + head;
    const float inv = 1.0f / Lsum;
    float* dst = z + rh * DC + 32 * cb + 4 * g;
#pragma unroll
    for (int j = 0; j < JP; ++j) {   // row groups 2 (jpbase + j) and 2 (jpbase + j) + 1
      *reinterpret_cast<f32x4*>(dst + 16 * (jpbase + j)) = acc[j][0] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * (jpbase + j) + 8) = acc[j][1] * inv;
    }
    if (lse != nullptr && cb == 0 && jpbase == 0 && g == 0) lse[rh] = (M + log2f(Lsum)) * kLn2;
  }
}

// Log-sum-exp merge of decode_attn_hsplit's head-major partials fused with the output
// projection o = W_UV,i z ("从零理解 MLA", section "矩阵吸收", output side), for mla_decode_step:
// the merge costs no launch of its own, and the weights stream in while the partials are read.
// One (query row, head, slice of the 128 outputs) per workgroup of 8 waves; kMergeSlices slices.
//   merge: the waves take the row's chunks round-robin (every chunk in one step); lane l reads
//   latent columns 8l .. 8l+7 (one 1 KB load of bf16 per wave and chunk) and keeps a running
//   maximum; the wave sums meet in LDS against the common maximum,
//   z = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k. A row computed as one chunk already has its
//   final z, written by the attention kernel, and is read back.
//   projection: wave w owns the OPW outputs (128 / kMergeSlices) y + OPW w + j of slice y, in
//   groups of 8; its lanes load
//   W_UV,i[v, 8l .. 8l+7] first, then dot them with z[8l .. 8l+7] and reduce across the wave exactly
//   as out_proj_gemv does (one 8-output butterfly per group), so o is bitwise what out_proj_gemv
//   makes of this z. Slice 0 writes z and lse. Every slice merges the partials again: one slice
//   would read them once, but at one query row (DeepSeek-V3 shape, 4K keys, 43 chunks) the decode
//   step measured 24.0 us with one slice against 22.5 us with two, the 256 workgroups hiding more
//   latency than the second read of 5.6 MB costs.
// grid (H, kMergeSlices, rows), 64 MERGE_WAVES threads.
constexpr int MERGE_WAVES = 8;
constexpr int kMergeSlices = 2;
__global__ void __launch_bounds__(64 * MERGE_WAVES)
    merge_heads_out_proj(const bf16* __restrict__ part_acc, const float* __restrict__ part_ml,
                         const int2* __restrict__ row_chunks, const bf16* __restrict__ w_uv, float* __restrict__ z,
                         float* __restrict__ lse, bf16* __restrict__ o) {
  constexpr int MW = MERGE_WAVES;
  constexpr int CU = kHsplitChunks / MW;   // chunks per step and wave: every chunk in one step
  constexpr int DV = 128;                  // d_v
  constexpr int OPW = DV / (kMergeSlices * MW);   // outputs per wave
  static_assert(OPW % 8 == 0, "whole groups of 8 outputs per wave");
  __shared__ f32x4 wacc[MW][2][64];
  __shared__ float wm[MW], wl[MW];
  __shared__ __attribute__((aligned(16))) float zs[DC];
  const int i = blockIdx.x, slice = blockIdx.y, bt = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const size_t rh = (size_t)bt * H + i;
  const int v0 = slice * (DV / kMergeSlices) + OPW * w;   // first output of this wave
  i32x4 wv[OPW];
  {
    const bf16* wp = w_uv + ((size_t)i * DV + v0) * DC + 8 * lane;
#pragma unroll
    for (int j = 0; j < OPW; ++j) wv[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp + (size_t)j * DC));
  }
  const int2 rc = row_chunks[bt];
  if (rc.y <= 1) {
    for (int c = t; c < DC; c += MW * 64) zs[c] = z[rh * DC + c];
  } else {
    const int base = rc.x, nck = rc.y;
    const bf16* src = part_acc + (size_t)base * PART_ELEMS + (size_t)i * DC + 8 * lane;
    const float2* ml = reinterpret_cast<const float2*>(part_ml) + (size_t)base * H + i;   // stride H per chunk
    float m_w = -INFINITY, Lsum = 0.0f;
    f32x4 a0 = {}, a1 = {};
    for (int k0 = w; k0 < nck; k0 += MW * CU) {
      i32x4 x[CU];
      float2 v[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int kk = k0 + MW * u;
        v[u] = make_float2(-INFINITY, 0.0f);
        if (kk < nck) {
          x[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src + (size_t)kk * PART_ELEMS));
          v[u] = ml[(size_t)kk * H];
        }
      }
      float mb = m_w;
#pragma unroll
      for (int u = 0; u < CU; ++u) mb = fmaxf(mb, v[u].x);
      const float a = exp2f(m_w - mb);   // 0 on the first step (m_w = -inf, mb finite)
      Lsum *= a;
      a0 *= a;
      a1 *= a;
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        if (k0 + MW * u < nck) {
          const float wk = exp2f(v[u].x - mb);
          Lsum = fmaf(wk, v[u].y, Lsum);
          f32x4 lo, hi;
          from_bf16x8(__builtin_bit_cast(bf16x8, x[u]), lo, hi);
          a0 += wk * lo;
          a1 += wk * hi;
        }
      }
      m_w = mb;
    }
    wacc[w][0][lane] = a0;
    wacc[w][1][lane] = a1;
    if (lane == 0) {
      wm[w] = m_w;
      wl[w] = Lsum;
    }
    __syncthreads();
    if (t < 64) {
      // wave 0 holds chunk 0, so M is finite; a wave without chunks weighs 2^-inf = 0
      float M = wm[0];
#pragma unroll
      for (int u = 1; u < MW; ++u) M = fmaxf(M, wm[u]);
      float e[MW];
      float L = 0.0f;
#pragma unroll
      for (int u = 0; u < MW; ++u) {
        e[u] = exp2f(wm[u] - M);
        L = fmaf(e[u], wl[u], L);
      }
      f32x4 acc0 = e[0] * wacc[0][0][t], acc1 = e[0] * wacc[0][1][t];
#pragma unroll
      for (int u = 1; u < MW; ++u) {
        acc0 += e[u] * wacc[u][0][t];
        acc1 += e[u] * wacc[u][1][t];
      }
      const float inv = 1.0f / L;
      const f32x4 z0 = acc0 * inv, z1 = acc1 * inv;
      const int c = 8 * t;   // this lane's 8 latent columns
      *reinterpret_cast<f32x4*>(&zs[c]) = z0;
      *reinterpret_cast<f32x4*>(&zs[c + 4]) = z1;
      if (slice == 0) {
        *reinterpret_cast<f32x4*>(z + rh * DC + c) = z0;
        *reinterpret_cast<f32x4*>(z + rh * DC + c + 4) = z1;
        if (lse != nullptr && t == 0) lse[rh] = (M + log2f(L)) * kLn2;
      }
    }
  }
  {
    __syncthreads();   // zs complete
    const f32x4 za = *reinterpret_cast<const f32x4*>(&zs[8 * lane]);
    const f32x4 zb = *reinterpret_cast<const f32x4*>(&zs[8 * lane + 4]);
#pragma unroll
    for (int gi = 0; gi < OPW / 8; ++gi) {
      float d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float wf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = (uint32_t)wv[8 * gi + j][e];
          wf[2 * e] = __uint_as_float(u << 16);
          wf[2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
        }
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
      // reduce-scatter (xor 32: 8 -> 4 outputs per lane, 16: 4 -> 2, 8: 2 -> 1), then xor 4, 2, 1
#pragma unroll
      for (int m = 32, n = 4; m >= 8; m >>= 1, n >>= 1) {
        const bool hi = lane & m;
#pragma unroll
        for (int j = 0; j < n; ++j) {
          const float send = hi ? d[j] : d[j + n];
          const float recv = __shfl_xor(send, m, 64);
          d[j] = (hi ? d[j + n] : d[j]) + recv;
        }
      }
      float s = d[0];
      s += __shfl_xor(s, 4, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 1, 64);
      // lane bits 5, 4, 3 -> output bits 2, 1, 0
      const int j = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
      if ((lane & 7) == 0) o[rh * DV + v0 + 8 * gi + j] = (bf16)s;
    }
  }
}

}  // namespace fast

bool attn_fast_supported(const LayerDims& L) {
  return L.n_heads == fast::H && L.d_latent == fast::DC && L.d_rope == fast::DR;
}

// workspace of the MFMA path: partial accumulators, (m, l) pairs, one (first slot, count) per row
size_t attn_fast_workspace_bytes(const SplitPlan& plan, int rows) {
  if (plan.fast_slots == 0) return 0;
  return (size_t)plan.fast_slots * ((size_t)fast::PART_ELEMS * sizeof(__bf16) + 2 * fast::H * sizeof(float)) +
         (size_t)rows * sizeof(int2);
}

void attn_fast_plan(int rows, int n_splits, int max_seq_len, SplitPlan* plan) {
  const int64_t max_tiles = ((int64_t)max_seq_len + fast::TILE - 1) / fast::TILE;
  if (n_splits == 0 && rows <= fast::kHsplitRows && rows * max_tiles <= fast::kHsplitMaxTiles) {
    plan->fast_mode = fast::HSPLIT;
    plan->fast_grid_x = 4 * fast::kHsplitChunks;
    plan->fast_slots = fast::kHsplitChunks;
  } else if (n_splits > 0) {
    plan->fast_mode = fast::FIXED;
    plan->fast_grid_x = plan->n_chunks;
    plan->fast_slots = plan->n_chunks > 1 ? rows * plan->n_chunks : 0;
  } else if (rows <= fast::kBalanceRows) {
    plan->fast_mode = fast::BALANCED;
    plan->fast_grid_x = fast::kBalanceGrid;
    plan->fast_slots = fast::kBalanceGrid;
  } else {
    plan->fast_mode = fast::PER_ROW;
    plan->fast_grid_x = rows;
    plan->fast_slots = 0;
  }
}

bool attn_fast_is_hsplit(const SplitPlan& plan) { return plan.fast_mode == fast::HSPLIT; }

namespace {
// workspace of the MFMA path: partial accumulators, then (m, l) pairs, then (first slot, count) per row
struct FastParts {
  __bf16* acc;
  float* ml;
  int2* row_chunks;
};
FastParts fast_parts(const SplitPlan& plan, void* workspace) {
  __bf16* acc = (__bf16*)workspace;
  float* ml = plan.fast_slots > 0 ? reinterpret_cast<float*>(acc + (size_t)plan.fast_slots * fast::PART_ELEMS) : nullptr;
  int2* rc = plan.fast_slots > 0 ? reinterpret_cast<int2*>(ml + (size_t)plan.fast_slots * 2 * fast::H) : nullptr;
  return FastParts{acc, ml, rc};
}
}  // namespace

hipError_t launch_merge_out_proj(const LayerDims& L, int rows, const SplitPlan& plan, const void* workspace,
                                 const void* w_uv, float* z, float* lse, void* o, hipStream_t stream) {
  (void)L;
  const FastParts P = fast_parts(plan, const_cast<void*>(workspace));
  hipLaunchKernelGGL(fast::merge_heads_out_proj, dim3(fast::H, fast::kMergeSlices, rows), dim3(64 * fast::MERGE_WAVES), 0, stream,
                     P.acc, P.ml, P.row_chunks, (const bf16*)w_uv, z, lse, (bf16*)o);
  return hipGetLastError();
}

hipError_t launch_attn_fast(const LayerDims& L, int batch, int n_q, const void* q_packed, const void* cache,
                            const int64_t* seq_off, const int32_t* seq_len, const SplitPlan& plan, void* workspace,
                            float* z, float* lse, hipStream_t stream, bool defer_merge) {
  const int rows = batch * n_q;
  const FastParts P = fast_parts(plan, workspace);
  __bf16* part_acc = P.acc;
  float* part_ml = P.ml;
  int2* row_chunks = P.row_chunks;
  static std::atomic<uint32_t> lds_set{0};
  {
    const hipError_t e = ensure_lds_limit(lds_set, {{(const void*)fast::decode_attn_fast, (int)sizeof(fast::Smem)},
                                                    {(const void*)fast::decode_attn_hsplit, (int)sizeof(fast::SmemH)}});
    if (e != hipSuccess) return e;
  }
  if (plan.fast_mode == fast::HSPLIT) {
    hipLaunchKernelGGL(fast::decode_attn_hsplit, dim3(plan.fast_grid_x), dim3(256), sizeof(fast::SmemH), stream,
                       (const bf16*)q_packed, (const bf16*)cache, seq_off, seq_len, n_q, rows,
                       L.softmax_scale * kLog2e, part_acc, part_ml, row_chunks, z, lse, defer_merge ? 1 : 0);
  } else {
    const dim3 grid(plan.fast_grid_x, plan.fast_mode == fast::FIXED ? rows : 1);
    hipLaunchKernelGGL(fast::decode_attn_fast, grid, dim3(256), sizeof(fast::Smem), stream, (const bf16*)q_packed,
                       (const bf16*)cache, seq_off, seq_len, n_q, rows, L.softmax_scale * kLog2e, plan.fast_mode,
                       plan.n_chunks, plan.chunk_len, part_acc, part_ml, row_chunks, z, lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.fast_slots == 0) return e;
  if (plan.fast_mode == fast::HSPLIT) {
    if (defer_merge) return hipSuccess;
    hipLaunchKernelGGL((fast::attn_merge_frag<1>), dim3(128, rows), dim3(256), 0, stream, part_acc, part_ml,
                       row_chunks, z, lse);
  } else if (rows <= 16) {   // few rows: two workgroups per (row, 32 x 32 block) to keep enough loads in flight
    hipLaunchKernelGGL((fast::attn_merge_frag<1>), dim3(128, rows), dim3(256), 0, stream, part_acc, part_ml,
                       row_chunks, z, lse);
  } else {
    hipLaunchKernelGGL((fast::attn_merge_frag<2>), dim3(64, rows), dim3(256), 0, stream, part_acc, part_ml,
                       row_chunks, z, lse);
  }
  return hipGetLastError();
}

}  // namespace mla

#ifdef MLA_PHASE_STAMPS
// Host side of the phase stamps (diagnostic build only; declared in include/mla_stamps.h).
#include "mla.h"
#include "mla_stamps.h"

extern "C" {

size_t mla_phase_stamps_bytes(void) { return sizeof(mla::fast::g_phase_stamps); }

int mla_phase_stamps_clear(void) {
  void* dev = nullptr;   // the device address of the array (its name in host code is only a stand-in)
  if (hipGetSymbolAddress(&dev, HIP_SYMBOL(mla::fast::g_phase_stamps)) != hipSuccess) return MLA_ERR_HIP;
  return hipMemset(dev, 0, sizeof(mla::fast::g_phase_stamps)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_phase_stamps_read(void* host_dst, size_t bytes) {
  if (host_dst == nullptr || bytes < sizeof(mla::fast::g_phase_stamps)) return MLA_ERR_INVALID_ARG;
  return hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(mla::fast::g_phase_stamps), sizeof(mla::fast::g_phase_stamps), 0,
                             hipMemcpyDeviceToHost) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

}  // extern "C"
#endif
